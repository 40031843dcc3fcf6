// q4k_dequant.hip — Q4_K super-blocks -> f32 [M][K] (gfx950).
//
// One thread per 16-byte quant word: the eight threads of a block together
// write its 256 outputs (1 KiB contiguous).  Each thread converts 16 low
// nibbles (sub-block 2g) and 16 high nibbles (sub-block 2g+1) with
// w = fma(q, d*sc, -dmin*m).  d*sc and dmin*m are exact in f32 (at most 17
// significant bits) and q*d*sc is exact inside the FMA, so the only rounding
// is the final one: the result is the exact value rounded to nearest-even,
// the same bits as any other evaluation order.
#include "q4k_device.hpp"
#include "q4k_internal.hpp"

namespace q4k {

namespace {

__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ w,
                                                      float *__restrict__ out, int64_t n_blocks,
                                                      int32_t nb, int64_t K) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t blk = t >> 3;
    if (blk >= n_blocks) return;
    const int c = (int)(t & 7);       // quant word 0..7
    const int g = c >> 1, h = c & 1;  // 32-byte group, half of the group
    const uint8_t *bp = w + blk * kBlockBytes;
    const uint4 hdr = ldg16(bp);
    const uint4 q = ldg16(bp + 16 + 16 * c);
    const float d = half_lo(hdr.x), dmin = half_hi(hdr.x);
    const Scales sc = unpack_scales(hdr.y, hdr.z, hdr.w);
    const float ds0 = d * scale_of(sc, 2 * g), dm0 = dmin * min_of(sc, 2 * g);
    const float ds1 = d * scale_of(sc, 2 * g + 1), dm1 = dmin * min_of(sc, 2 * g + 1);

    const int64_t row = blk / nb;
    const int64_t col0 = (blk - row * nb) * 256 + 64 * g + 16 * h;
    float4 *lo_out = reinterpret_cast<float4 *>(out + row * K + col0);
    float4 *hi_out = reinterpret_cast<float4 *>(out + row * K + col0 + 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t v = word_of(q, i);
        const uint32_t lo = and_mask(v, 0x0F0F0F0Fu);
        const uint32_t hi = and_mask(v >> 4, 0x0F0F0F0Fu);
        lo_out[i] = make_float4(fmaf(ubyte(lo, 0), ds0, -dm0), fmaf(ubyte(lo, 1), ds0, -dm0),
                                fmaf(ubyte(lo, 2), ds0, -dm0), fmaf(ubyte(lo, 3), ds0, -dm0));
        hi_out[i] = make_float4(fmaf(ubyte(hi, 0), ds1, -dm1), fmaf(ubyte(hi, 1), ds1, -dm1),
                                fmaf(ubyte(hi, 2), ds1, -dm1), fmaf(ubyte(hi, 3), ds1, -dm1));
    }
}

}  // namespace

int launch_dequant(const uint8_t *w, float *out, int64_t M, int64_t K, hipStream_t stream) {
    const int64_t n_blocks = M * (K / 256);
    const int64_t threads = n_blocks * 8;
    const int64_t groups = (threads + 255) / 256;
    if (groups == 0) return Q4K_OK;
    if (groups > 0x7FFFFFFF) return fail(Q4K_EUNSUPPORTED, "dequant: matrix too large");
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)groups), dim3(256), 0, stream, w, out,
                       n_blocks, (int32_t)(K / 256), K);
    Q4K_HIP(hipGetLastError());
    return Q4K_OK;
}

}  // namespace q4k
