// Pieces shared by the two product kernels (small-M streaming and large-M tiled).
#pragma once

#include "device_common.h"
#include "hts_internal.h"

namespace hts {

// k-order of the dense substeps.  Within each 64-wide slice of a tile, dense
// substep u = 2s + v (s = slice, v = 0/1) gives lane group g (lanes 16g..16g+15)
// the 8 consecutive k starting at koff(u, g), for the weight operand and the X
// operand alike (any k order shared by both operands leaves the sum unchanged).
//   SMFMAC order: koff = 64s + 32v + 8g  -- the two X chunks of slice s are then
//     exactly the B operand of the 16x16x64 SMFMAC for that slice.
//   expansion order: koff = 64s + 16g + 8v -- lane group g then covers the same
//     16 dense k as the stored values it expands.
template <int SP>
__device__ __forceinline__ constexpr int koff(int u, int g) {
    return SP == SPARSE_SMFMAC ? 64 * (u >> 1) + 32 * (u & 1) + 8 * g
                               : 64 * (u >> 1) + 16 * g + 8 * (u & 1);
}

// Store 1 or 4 consecutive outputs of one Y row with rounding to y_dtype.
__device__ __forceinline__ void store_y1(void* Y, int64_t off, int32_t y_dtype, float v) {
    if (y_dtype == HTS_F32) {
        reinterpret_cast<float*>(Y)[off] = v;
    } else if (y_dtype == HTS_BF16) {
        reinterpret_cast<uint16_t*>(Y)[off] = (uint16_t)narrow_bf16(v);
    } else {
        reinterpret_cast<uint16_t*>(Y)[off] = (uint16_t)narrow_f16(v);
    }
}

// Gated output: silu(g) * v with silu(x) = x / (1 + e^-x), g = G[off] in the output type (fp32
// arithmetic, one rounding when the result is stored).
__device__ __forceinline__ float gate_value(const void* G, int64_t off, int32_t dt) {
    if (dt == HTS_F32) return reinterpret_cast<const float*>(G)[off];
    const uint32_t b = reinterpret_cast<const uint16_t*>(G)[off];
    return dt == HTS_BF16 ? widen<BF16T>(b) : widen<F16T>(b);
}
__device__ __forceinline__ float silu_times(float g, float v) { return g / (1.0f + expf(-g)) * v; }
// Four consecutive gate values G[off .. off+3] in one load (off is a multiple of 4 and G is
// 16-byte aligned: 8 bytes for 16-bit types, 16 for fp32).
__device__ __forceinline__ f32x4 load_gate4(const void* G, int64_t off, int32_t dt) {
    if (dt == HTS_F32) return *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(G) + off);
    const uint2 b = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(G) + off);
    const uint32_t h[4] = {b.x & 0xFFFFu, b.x >> 16, b.y & 0xFFFFu, b.y >> 16};
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = dt == HTS_BF16 ? widen<BF16T>(h[e]) : widen<F16T>(h[e]);
    return r;
}
__device__ __forceinline__ f32x4 silu_times4(f32x4 g, f32x4 v) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = silu_times(g[e], v[e]);
    return r;
}

__device__ __forceinline__ void store_y4(void* Y, int64_t off, int32_t y_dtype, f32x4 v) {
    if (y_dtype == HTS_F32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(Y) + off) = v;
    } else {
        uint32_t b[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = (y_dtype == HTS_BF16) ? narrow_bf16(v[r]) : narrow_f16(v[r]);
        uint2 p = {b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(Y) + off) = p;
    }
}

}  // namespace hts
