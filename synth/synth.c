/*
 * synth.c — seeded synthetic inputs for the Q4_K matmul path.
 *
 * This module only *produces bytes*: it holds none of the arithmetic that the
 * matmul path or its CPU reference computes (no dequantisation, no dot
 * products).  Both the HIP path and the CPU reference consume the bytes that
 * it writes, so the two never generate independently.
 *
 * Random source: SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014), used in its
 * counter form: word i of the stream keyed by `key` is the mixing function
 * applied to key + (i+1)*gamma, which equals the (i+1)-th output of the
 * sequential generator seeded with `key`.  Any word can therefore be produced
 * independently, so the OpenMP loops below give the same bytes for any thread
 * count.
 *
 * Q4_K super-block stream (144 bytes per block, 20 words per block):
 *   word 20b+0 -> d    : U(lo, hi) in double, rounded to IEEE binary16 (RNE)
 *   word 20b+1 -> dmin : U(lo, hi) in double, rounded to IEEE binary16 (RNE)
 *   words 20b+2, 20b+3 -> the 12 packed scale/min bytes (first 12 of 16 bytes)
 *   words 20b+4 .. 20b+19 -> the 128 nibble bytes
 * Uniform bytes give uniform 6-bit scales/mins and uniform nibbles under any
 * bijective packing, so the distribution does not depend on the layout.
 *
 * Q8_0 block stream: see synth_q8_0_blocks.
 * Q6_K block stream: see synth_q6_k_blocks.
 *
 * Normal activations: Box–Muller (G. E. P. Box, M. E. Muller, 1958) on the
 * word pair (2i, 2i+1), computed in double and rounded once to f32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_word(uint64_t key, uint64_t i) {
    uint64_t z = key + (i + 1u) * SM64_GAMMA;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* 53-bit uniform in [0, 1). */
static inline double u01(uint64_t w) { return (double)(w >> 11) * 0x1.0p-53; }

/* Round a finite, positive double that lies in the binary16 normal range to
 * the nearest binary16 (ties to even).  Returns the bit pattern, or 0xFFFF if
 * the value is outside the range this generator produces. */
static uint16_t half_bits_rne(double v) {
    if (!(v >= 0x1.0p-14 && v < 65504.0)) return 0xFFFF;
    int e;
    double fr = frexp(v, &e);          /* v = fr * 2^e, fr in [0.5, 1) */
    double sig = nearbyint(ldexp(fr, 11)); /* 11-bit significand, RNE */
    if (sig == 2048.0) { sig = 1024.0; e += 1; }
    int biased = (e - 1) + 15;
    if (biased < 1 || biased > 30) return 0xFFFF;
    return (uint16_t)((biased << 10) | ((int)sig - 1024));
}

uint64_t synth_word(uint64_t key, uint64_t i) { return sm64_word(key, i); }

uint16_t synth_half_bits(double v) { return half_bits_rne(v); }

/* Write `nblocks` super-blocks, starting at block index `block0` of the stream
 * keyed by `key`, to `out` (nblocks*144 bytes).  Returns 0, or -1 if a d/dmin
 * draw fell outside the binary16 normal range (bad lo/hi). */
int synth_q4k_blocks(uint64_t key, uint64_t block0, uint64_t nblocks,
                     uint8_t *out, double lo, double hi) {
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t bi = 0; bi < (int64_t)nblocks; ++bi) {
        uint64_t b = block0 + (uint64_t)bi;
        uint8_t *p = out + (uint64_t)bi * 144u;
        uint64_t base = b * 20u;
        uint16_t hd = half_bits_rne(lo + (hi - lo) * u01(sm64_word(key, base + 0)));
        uint16_t hm = half_bits_rne(lo + (hi - lo) * u01(sm64_word(key, base + 1)));
        if (hd == 0xFFFF || hm == 0xFFFF) bad = 1;
        p[0] = (uint8_t)(hd & 0xFF); p[1] = (uint8_t)(hd >> 8);
        p[2] = (uint8_t)(hm & 0xFF); p[3] = (uint8_t)(hm >> 8);
        uint8_t tmp[16];
        uint64_t w2 = sm64_word(key, base + 2), w3 = sm64_word(key, base + 3);
        memcpy(tmp, &w2, 8); memcpy(tmp + 8, &w3, 8);
        memcpy(p + 4, tmp, 12);
        for (int j = 0; j < 16; ++j) {
            uint64_t w = sm64_word(key, base + 4 + (uint64_t)j);
            memcpy(p + 16 + 8 * j, &w, 8);
        }
    }
    return bad ? -1 : 0;
}

/* Q8_0 block stream (34 bytes per block, 5 words per block):
 *   word 5b+0 -> d : U(lo, hi) in double, rounded to IEEE binary16 (RNE)
 *   words 5b+1 .. 5b+4 -> the 32 quant bytes (uniform over all 256 values). */
int synth_q8_0_blocks(uint64_t key, uint64_t block0, uint64_t nblocks,
                      uint8_t *out, double lo, double hi) {
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t bi = 0; bi < (int64_t)nblocks; ++bi) {
        uint64_t b = block0 + (uint64_t)bi;
        uint8_t *p = out + (uint64_t)bi * 34u;
        uint64_t base = b * 5u;
        uint16_t hd = half_bits_rne(lo + (hi - lo) * u01(sm64_word(key, base + 0)));
        if (hd == 0xFFFF) bad = 1;
        p[0] = (uint8_t)(hd & 0xFF); p[1] = (uint8_t)(hd >> 8);
        for (int j = 0; j < 4; ++j) {
            uint64_t w = sm64_word(key, base + 1 + (uint64_t)j);
            memcpy(p + 2 + 8 * j, &w, 8);
        }
    }
    return bad ? -1 : 0;
}

/* n standard-normal f32 values from the stream keyed by `key`. */
/* Q6_K block stream: per block b, word 27b gives d = U(lo, hi) rounded to
 * binary16 (stored in the last two bytes), and words 27b+1 .. 27b+26 give
 * the 208 bytes before it (quant low bits, quant high bits and the sixteen
 * int8 scales, all uniform), eight bytes per word, the last word's final
 * six bytes unused. */
int synth_q6_k_blocks(uint64_t key, uint64_t block0, uint64_t nblocks,
                      uint8_t *out, double lo, double hi) {
    int bad = 0;
    #pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t bi = 0; bi < (int64_t)nblocks; ++bi) {
        uint64_t b = block0 + (uint64_t)bi;
        uint8_t *p = out + (uint64_t)bi * 210u;
        uint64_t base = b * 27u;
        uint16_t hd = half_bits_rne(lo + (hi - lo) * u01(sm64_word(key, base + 0)));
        if (hd == 0xFFFF) bad = 1;
        for (int j = 0; j < 26; ++j) {
            uint64_t w = sm64_word(key, base + 1 + (uint64_t)j);
            memcpy(p + 8 * j, &w, 8);
        }
        p[208] = (uint8_t)(hd & 0xFF); p[209] = (uint8_t)(hd >> 8);
    }
    return bad ? -1 : 0;
}

void synth_normal_f32(uint64_t key, uint64_t n, float *out) {
    uint64_t pairs = (n + 1) / 2;
    #pragma omp parallel for schedule(static)
    for (int64_t pi = 0; pi < (int64_t)pairs; ++pi) {
        uint64_t i = (uint64_t)pi;
        double u1 = ((double)(sm64_word(key, 2 * i) >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
        double u2 = u01(sm64_word(key, 2 * i + 1));
        double r = sqrt(-2.0 * log(u1));
        double a = 6.283185307179586476925286766559 * u2;
        out[2 * i] = (float)(r * cos(a));
        if (2 * i + 1 < n) out[2 * i + 1] = (float)(r * sin(a));
    }
}

/* n raw bytes from the stream keyed by `key` (little-endian words). */
void synth_bytes(uint64_t key, uint64_t n, uint8_t *out) {
    uint64_t words = (n + 7) / 8;
    #pragma omp parallel for schedule(static)
    for (int64_t wi = 0; wi < (int64_t)words; ++wi) {
        uint64_t w = sm64_word(key, (uint64_t)wi);
        uint64_t off = (uint64_t)wi * 8u;
        uint64_t take = (n - off) < 8 ? (n - off) : 8;
        memcpy(out + off, &w, take);
    }
}
