// Device-side helpers for gfx950 (CDNA4): 16-bit element handling and the
// dense / sparse matrix-core instructions used by the product kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hts {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

// Element-type tags.  BF16 = bfloat16, F16 = IEEE binary16.
struct BF16T { static constexpr int id = 1; };
struct F16T { static constexpr int id = 0; };

// Exact widening of one 16-bit pattern to float.
template <typename T> __device__ __forceinline__ float widen(uint32_t bits);
template <> __device__ __forceinline__ float widen<BF16T>(uint32_t bits) {
    return __uint_as_float(bits << 16);
}
template <> __device__ __forceinline__ float widen<F16T>(uint32_t bits) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits);
    return (float)h;
}

// Round-to-nearest-even narrowing of a float (finite or not) to a 16-bit pattern.
__device__ __forceinline__ uint32_t narrow_bf16(float f) {
    __bf16 b = (__bf16)f;                      // RNE conversion on gfx950
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t narrow_f16(float f) {
    _Float16 h = (_Float16)f;                  // RNE conversion
    return __builtin_bit_cast(uint16_t, h);
}

// Dense 16x16x32 MFMA: A[16][32] x B[32][16] -> C[16][16], fp32 accumulate.
// Operand lanes: A lane (i + 16h) holds A[i][8h .. 8h+7]; B lane (j + 16q) holds
// B[8q .. 8q+7][j]; C lane (j + 16q) holds C[4q .. 4q+3][j].
template <typename T> __device__ __forceinline__ f32x4 mfma_dense(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma_dense<BF16T>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma_dense<F16T>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Sparse 16x16x64 MFMA (SMFMAC): A is 16 x 64 with two of every four entries
// stored.  A lane (i + 16h) holds the 8 stored values of row i for dense
// k in [16h, 16h+16): value v belongs to group v/2 and sits at position
// 4*(v/2) + idx_v, idx_v = bits [2v+1:2v] of the selected 16-bit index half
// (ABID = 0: low half, 1: high half).  B lane (j + 16q) holds B[8q+e][j] for
// e < 8 and B[32+8q+(e-8)][j] for e >= 8.  C as for the dense instruction.
// (Lane layout measured on gfx950 with one-hot operands.)
template <typename T, int ABID>
__device__ __forceinline__ f32x4 mfma_sparse(u32x4 a, u32x8 b, uint32_t idx, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma_sparse<BF16T, 0>(u32x4 a, u32x8 b, uint32_t idx, f32x4 c) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x16, b), c, (int)idx, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_sparse<BF16T, 1>(u32x4 a, u32x8 b, uint32_t idx, f32x4 c) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x16, b), c, (int)idx, 0, 1);
}
template <>
__device__ __forceinline__ f32x4 mfma_sparse<F16T, 0>(u32x4 a, u32x8 b, uint32_t idx, f32x4 c) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x16, b), c, (int)idx, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_sparse<F16T, 1>(u32x4 a, u32x8 b, uint32_t idx, f32x4 c) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x16, b), c, (int)idx, 0, 1);
}

// ---- 8-bit OCP E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits) ----
struct FP8T { static constexpr int id = 3; };

// Exact value of one E4M3 byte (every E4M3 value is a binary32 value); the NaN patterns 0x7F /
// 0xFF decode as 480 -- their products are unspecified.
__device__ __forceinline__ float widen_e4m3(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -mag : mag;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Dense 16x16x32 8-bit MFMA (E4M3 x E4M3): lane (i + 16g) holds 8 values of row i of A for the
// instruction's k slot g, B lane (j + 16q) the 8 values of column j for slot q.  Any one k order
// shared by A and B gives the same product, so the data keeps the chunk layout of the sparse
// 16x16x128 instruction below (lane group g: 16-byte chunks g and 4 + g of a 128-byte row) and
// each 16-byte chunk feeds two of these instructions, one per 8-byte half: every k is used once.
__device__ __forceinline__ f32x4 mfma_fp8_dense32(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8((long)__builtin_bit_cast(uint64_t, a),
                                                      (long)__builtin_bit_cast(uint64_t, b), c, 0, 0, 0);
}
// One 16-byte chunk per lane group of A and B: two 8-bit 16x16x32 products.
template <>
__device__ __forceinline__ f32x4 mfma_dense<FP8T>(u32x4 a, u32x4 b, f32x4 c) {
    c = mfma_fp8_dense32(uint2{a[0], a[1]}, uint2{b[0], b[1]}, c);
    return mfma_fp8_dense32(uint2{a[2], a[3]}, uint2{b[2], b[3]}, c);
}

// Dense 16x16x128 8-bit MFMA (the f8f6f4 form, E4M3 for A and B, unit block scales: E8M0 exponent
// 127): lane (i + 16g) holds 32 values of row i of A and of column i of B.  Fed with the chunk
// layout of the sparse 16x16x128 instruction below (16-byte chunks g and 4 + g of the 128-byte row)
// for both operands, every k of the 128 is used once; one instruction does the work of four
// 16x16x32 ones at twice their rate.  It takes twice the cycles of the sparse instruction below:
// where one accumulator is written by both on the two arms of a branch, the compiler has read it
// after the join with the sparse instruction's wait states (stale sums), so callers keep the two
// in separate loops or separate accumulators.
__device__ __forceinline__ f32x4 mfma_fp8_dense128(u32x8 a, u32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(__builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, b),
                                                            c, 0, 0, 0, 127, 0, 127);
}

// Sparse 16x16x128 8-bit SMFMAC: A lane (i + 16h) holds the 16 stored values of row i for dense
// k in [32h, 32h+32): value v belongs to group v/2 at position 4*(v/2) + idx_v, idx_v = bits
// [2v+1:2v] of the whole 32-bit index.  B lane (j + 16q) holds B[16q+e][j] for e < 16 and
// B[64+16q+(e-16)][j] for e >= 16.  (Lane layouts measured on gfx950 with random small-integer
// operands against every candidate order.)
__device__ __forceinline__ f32x4 mfma_fp8_sparse(u32x4 a, u32x8 b, uint32_t idx, f32x4 c) {
    return __builtin_amdgcn_smfmac_f32_16x16x128_fp8_fp8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x8, b), c,
                                                        (int)idx, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma_sparse<FP8T, 0>(u32x4 a, u32x8 b, uint32_t idx, f32x4 c) {
    return mfma_fp8_sparse(a, b, idx, c);
}

// Bytes per element and K elements per 128-byte row slice of the tiled kernels.
template <typename T> struct Elem { static constexpr int bytes = 2; };
template <> struct Elem<FP8T> { static constexpr int bytes = 1; };

__device__ __forceinline__ u32x4 lo4(u32x8 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ u32x4 hi4(u32x8 v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }
__device__ __forceinline__ u32x8 cat8(u32x4 a, u32x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Expand two 2:4 groups (4 stored 16-bit values in `v`, codes in the low byte
// of `nib`: group 0 bits 0..3, group 1 bits 4..7) into 8 dense 16-bit values.
__device__ __forceinline__ u32x4 expand_two_groups(uint2 v, uint32_t nib) {
    uint32_t vals[4] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16};
    uint32_t out[8];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        uint32_t code = (nib >> (4 * g)) & 0xFu;
        uint32_t i0 = code & 3u, i1 = code >> 2;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t x = (i0 == (uint32_t)p) ? vals[2 * g] : 0u;
            x = (i1 == (uint32_t)p) ? vals[2 * g + 1] : x;
            out[4 * g + p] = x;
        }
    }
    u32x4 r = {out[0] | (out[1] << 16), out[2] | (out[3] << 16), out[4] | (out[5] << 16),
               out[6] | (out[7] << 16)};
    return r;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace hts
