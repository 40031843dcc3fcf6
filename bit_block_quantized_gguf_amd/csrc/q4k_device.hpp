// q4k_device.hpp — gfx950 device helpers for Q4_K super-blocks.
//
// A super-block is 144 bytes = nine 16-byte words: word 0 carries d, dmin and
// the 12 packed scale/min bytes; words 1..8 carry the 128 quant bytes.  In
// 32-byte group g (words 2g+1, 2g+2), byte l holds weight 64g+l in its low
// nibble (sub-block 2g) and weight 64g+32+l in its high nibble (sub-block
// 2g+1).  Weight value: d*sc[j]*q - dmin*m[j] (public GGUF Q4_K convention).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace q4k {

constexpr int kBlockWeights = 256;
constexpr int kBlockBytes = 144;
constexpr int kWave = 64;

// Activation pointer in the constant address space: loads through it with a
// wave-uniform address become scalar loads, so an activation value reaches
// the FMA as an SGPR operand and costs no vector-memory bandwidth.
typedef const float __attribute__((address_space(4))) cfloat;

__device__ __forceinline__ cfloat *as_const(const float *p) { return (cfloat *)p; }

// Bitwise AND hidden from the optimiser.  With a visible mask the compiler
// folds `(v & 0x0F0F0F0F) >> 8 & 0xFF` into a 4-bit field extract followed by
// a byte-0 conversion (two instructions per weight); behind this barrier every
// weight converts with a single v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t and_mask(uint32_t v, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(m), "v"(v));
    return r;
}

// (v & m) | c in one v_and_or_b32, hidden from the optimiser like and_mask.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t m, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(v), "v"(m), "v"(c));
    return r;
}

__device__ __forceinline__ float ubyte(uint32_t v, int b) {
    return (float)((v >> (8 * b)) & 0xFFu);
}

__device__ __forceinline__ float half_lo(uint32_t v) {
    return __half2float(__ushort_as_half((unsigned short)(v & 0xFFFFu)));
}
__device__ __forceinline__ float half_hi(uint32_t v) {
    return __half2float(__ushort_as_half((unsigned short)(v >> 16)));
}

// Header word -> four dwords whose bytes are the sixteen 6-bit fields:
//   scl: sc[0..3], sch: sc[4..7], mnl: m[0..3], mnh: m[4..7].
// s[0..3] (A) low six bits are sc[0..3], top two bits are bits 4-5 of
// sc[4..7]; s[4..7] (B) likewise for m; s[8..11] (C) low nibbles are bits
// 0-3 of sc[4..7], high nibbles bits 0-3 of m[4..7].
struct Scales {
    uint32_t scl, sch, mnl, mnh;
};

__device__ __forceinline__ Scales unpack_scales(uint32_t A, uint32_t B, uint32_t C) {
    Scales s;
    s.scl = A & 0x3F3F3F3Fu;
    s.mnl = B & 0x3F3F3F3Fu;
    s.sch = (C & 0x0F0F0F0Fu) | ((A >> 2) & 0x30303030u);
    s.mnh = ((C >> 4) & 0x0F0F0F0Fu) | ((B >> 2) & 0x30303030u);
    return s;
}

__device__ __forceinline__ float scale_of(const Scales &s, int j) {
    return j < 4 ? ubyte(s.scl, j) : ubyte(s.sch, j - 4);
}
__device__ __forceinline__ float min_of(const Scales &s, int j) {
    return j < 4 ? ubyte(s.mnl, j) : ubyte(s.mnh, j - 4);
}

__device__ __forceinline__ uint4 ldg16(const uint8_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

}  // namespace q4k
