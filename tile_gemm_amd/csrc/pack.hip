// Pack / unpack of a tile-level hybrid (dense / 2:4) weight on gfx950.
//
// One workgroup per tile (page "PATCH: Learnable Tile-level Hybrid Sparsity for
// LLMs", section 2: the dense / 2:4 decision is made per tile).  Each thread
// handles 32 consecutive weights of one tile row: four 16-byte loads, and either
// a raw copy (dense tile) or eight 2-of-4 selections producing 16 kept values
// and one 32-bit metadata word (2:4 tile).  The pass is bound by HBM bandwidth:
// it reads W once and writes the packed bytes once.
#include "device_common.h"
#include "hts_internal.h"

namespace hts {
namespace {

constexpr int kPackThreads = 256;

// Score of one weight: |w| as binary32, times the column scale when given
// (a single IEEE multiply: nothing to contract).
template <typename T>
__device__ __forceinline__ float score(uint32_t bits, const float* cs, int64_t k) {
    float a = fabsf(widen<T>(bits));
    return cs ? a * cs[k] : a;
}

// Kept pair of a group: weight i is kept when fewer than two others beat it,
// j beating i when s_j > s_i, or s_j == s_i with j < i.
__device__ __forceinline__ void pick_two(const float s[4], uint32_t& i0, uint32_t& i1) {
    bool keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int rank = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j == i) continue;
            rank += (s[j] > s[i]) || (s[j] == s[i] && j < i);
        }
        keep[i] = rank < 2;
    }
    i0 = keep[0] ? 0u : (keep[1] ? 1u : 2u);
    i1 = keep[3] ? 3u : (keep[2] ? 2u : 1u);
}

// MASKED: the 2:4 pairs come from an element mask (PATCH page, section 2, variants: the
// PATCH-Tile variant freezes 2:4 patterns from a one-shot method): the score of a weight is 1
// where the mask byte is nonzero, else 0, under the same rank rule, so a group marking exactly
// two weights keeps those two.  Groups marking another number are counted into *malformed.
template <typename T, bool MASKED>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const hts_tile* __restrict__ index, int64_t Tk, int bn, int bk,
    const uint16_t* __restrict__ W, int64_t ldw, const float* __restrict__ cs,
    const uint8_t* __restrict__ mask, int64_t ldm, uint32_t* __restrict__ malformed,
    uint16_t* __restrict__ values, uint32_t* __restrict__ meta) {
    const int64_t t = blockIdx.x;
    uint32_t bad = 0;
    const hts_tile e = index[t];
    const int64_t tn = t / Tk, tk = t % Tk;
    const int wpr = bk / 32;                       // 32-weight chunks per tile row
    const int items = bn * wpr;
    for (int it = threadIdx.x; it < items; it += kPackThreads) {
        const int r = it / wpr, w = it % wpr;
        const int64_t k0 = tk * bk + 32 * w;
        const uint16_t* src = W + (tn * bn + r) * ldw + k0;
        u32x4 q[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = ld16(src + 8 * c);
        if (e.type == HTS_TILE_DENSE) {
            uint16_t* dst = values + e.val_off + (int64_t)r * bk + 32 * w;
#pragma unroll
            for (int c = 0; c < 4; ++c) st16(dst + 8 * c, q[c]);
            continue;
        }
        uint32_t kept[8];   // 16 kept 16-bit values, two per word
        uint32_t word = 0;
        u32x4 mk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};   // 32 mask bytes of the chunk
        if (MASKED) {
            const uint8_t* msrc = mask + (tn * bn + r) * ldm + k0;
            mk[0] = *reinterpret_cast<const u32x4*>(msrc);
            mk[1] = *reinterpret_cast<const u32x4*>(msrc + 16);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            // group g = weights 4g..4g+3 of this chunk = dwords 2g, 2g+1
            const uint32_t d0 = q[g / 2][(2 * g) % 4], d1 = q[g / 2][(2 * g + 1) % 4];
            const uint32_t b[4] = {d0 & 0xFFFFu, d0 >> 16, d1 & 0xFFFFu, d1 >> 16};
            float s[4];
            if (MASKED) {
                const uint32_t mw = mk[g / 4][g % 4];            // mask bytes of weights 4g..4g+3
                int marked = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool on = ((mw >> (8 * i)) & 0xFFu) != 0u;
                    s[i] = on ? 1.0f : 0.0f;
                    marked += on;
                }
                bad += marked != 2;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) s[i] = score<T>(b[i], cs, k0 + 4 * g + i);
            }
            uint32_t i0, i1;
            pick_two(s, i0, i1);
            uint32_t v0 = b[0], v1 = b[1];
            v0 = (i0 == 1u) ? b[1] : v0;
            v0 = (i0 == 2u) ? b[2] : v0;
            v1 = (i1 == 2u) ? b[2] : v1;
            v1 = (i1 == 3u) ? b[3] : v1;
            kept[g] = v0 | (v1 << 16);
            word |= (i0 | (i1 << 2)) << (4 * g);
        }
        uint16_t* dst = values + e.val_off + (int64_t)r * (bk / 2) + 16 * w;
        u32x4 o0 = {kept[0], kept[1], kept[2], kept[3]};
        u32x4 o1 = {kept[4], kept[5], kept[6], kept[7]};
        st16(dst, o0);
        st16(dst + 8, o1);
        meta[e.meta_off + (int64_t)r * wpr + w] = word;
    }
    if (MASKED && malformed && bad) atomicAdd(malformed, bad);
}

// The same pass for 8-bit E4M3 weights: a thread takes 32 consecutive bytes of a tile row (two
// 16-byte loads); a 2:4 chunk becomes 16 kept bytes (one 16-byte store) and the same 32-bit code
// word as above.  The score is |w| decoded exactly (times the column scale when given).
template <bool MASKED>
__global__ __launch_bounds__(kPackThreads) void pack8_kernel(
    const hts_tile* __restrict__ index, int64_t Tk, int bn, int bk,
    const uint8_t* __restrict__ W, int64_t ldw, const float* __restrict__ cs,
    const uint8_t* __restrict__ mask, int64_t ldm, uint32_t* __restrict__ malformed,
    uint8_t* __restrict__ values, uint32_t* __restrict__ meta) {
    const int64_t t = blockIdx.x;
    uint32_t bad = 0;
    const hts_tile e = index[t];
    const int64_t tn = t / Tk, tk = t % Tk;
    const int wpr = bk / 32;
    const int items = bn * wpr;
    for (int it = threadIdx.x; it < items; it += kPackThreads) {
        const int r = it / wpr, w = it % wpr;
        const int64_t k0 = tk * bk + 32 * w;
        const uint8_t* src = W + (tn * bn + r) * ldw + k0;
        const u32x4 q0 = ld16(src), q1 = ld16(src + 16);
        if (e.type == HTS_TILE_DENSE) {
            uint8_t* dst = values + e.val_off + (int64_t)r * bk + 32 * w;
            st16(dst, q0);
            st16(dst + 16, q1);
            continue;
        }
        const uint32_t d[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};   // group g = d[g]
        u32x4 mk[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
        if (MASKED) {
            const uint8_t* msrc = mask + (tn * bn + r) * ldm + k0;
            mk[0] = *reinterpret_cast<const u32x4*>(msrc);
            mk[1] = *reinterpret_cast<const u32x4*>(msrc + 16);
        }
        uint32_t kept[8];   // kept pair of group g: low byte = lower index
        uint32_t word = 0;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const uint32_t b[4] = {d[g] & 0xFFu, (d[g] >> 8) & 0xFFu, (d[g] >> 16) & 0xFFu, d[g] >> 24};
            float sc[4];
            if (MASKED) {
                const uint32_t mw = mk[g / 4][g % 4];
                int marked = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool on = ((mw >> (8 * i)) & 0xFFu) != 0u;
                    sc[i] = on ? 1.0f : 0.0f;
                    marked += on;
                }
                bad += marked != 2;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = fabsf(widen_e4m3(b[i]));
                    sc[i] = cs ? a * cs[k0 + 4 * g + i] : a;
                }
            }
            uint32_t i0, i1;
            pick_two(sc, i0, i1);
            uint32_t v0 = b[0], v1 = b[1];
            v0 = (i0 == 1u) ? b[1] : v0;
            v0 = (i0 == 2u) ? b[2] : v0;
            v1 = (i1 == 2u) ? b[2] : v1;
            v1 = (i1 == 3u) ? b[3] : v1;
            kept[g] = v0 | (v1 << 8);
            word |= (i0 | (i1 << 2)) << (4 * g);
        }
        uint8_t* dst = values + e.val_off + (int64_t)r * (bk / 2) + 16 * w;
        st16(dst, u32x4{kept[0] | (kept[1] << 16), kept[2] | (kept[3] << 16), kept[4] | (kept[5] << 16),
                        kept[6] | (kept[7] << 16)});
        meta[e.meta_off + (int64_t)r * wpr + w] = word;
    }
    if (MASKED && malformed && bad) atomicAdd(malformed, bad);
}

__global__ void zero_counter(uint32_t* c) { *c = 0u; }

__global__ __launch_bounds__(kPackThreads) void unpack_kernel(
    const hts_tile* __restrict__ index, int64_t Tk, int bn, int bk,
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ meta,
    uint16_t* __restrict__ W, int64_t ldw) {
    const int64_t t = blockIdx.x;
    const hts_tile e = index[t];
    const int64_t tn = t / Tk, tk = t % Tk;
    const int wpr = bk / 32;
    const int items = bn * wpr;
    for (int it = threadIdx.x; it < items; it += kPackThreads) {
        const int r = it / wpr, w = it % wpr;
        uint16_t* dst = W + (tn * bn + r) * ldw + tk * bk + 32 * w;
        if (e.type == HTS_TILE_DENSE) {
            const uint16_t* src = values + e.val_off + (int64_t)r * bk + 32 * w;
#pragma unroll
            for (int c = 0; c < 4; ++c) st16(dst + 8 * c, ld16(src + 8 * c));
            continue;
        }
        const uint16_t* src = values + e.val_off + (int64_t)r * (bk / 2) + 16 * w;
        const u32x4 a = ld16(src), b = ld16(src + 8);
        const uint32_t word = meta[e.meta_off + (int64_t)r * wpr + w];
        const uint32_t kv[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
        for (int c = 0; c < 4; ++c) {   // output chunk c = groups 2c, 2c+1
            uint2 v = {kv[2 * c], kv[2 * c + 1]};
            st16(dst + 8 * c, expand_two_groups(v, (word >> (8 * c)) & 0xFFu));
        }
    }
}

__global__ __launch_bounds__(kPackThreads) void unpack8_kernel(
    const hts_tile* __restrict__ index, int64_t Tk, int bn, int bk,
    const uint8_t* __restrict__ values, const uint32_t* __restrict__ meta,
    uint8_t* __restrict__ W, int64_t ldw) {
    const int64_t t = blockIdx.x;
    const hts_tile e = index[t];
    const int64_t tn = t / Tk, tk = t % Tk;
    const int wpr = bk / 32;
    const int items = bn * wpr;
    for (int it = threadIdx.x; it < items; it += kPackThreads) {
        const int r = it / wpr, w = it % wpr;
        uint8_t* dst = W + (tn * bn + r) * ldw + tk * bk + 32 * w;
        if (e.type == HTS_TILE_DENSE) {
            const uint8_t* src = values + e.val_off + (int64_t)r * bk + 32 * w;
            st16(dst, ld16(src));
            st16(dst + 16, ld16(src + 16));
            continue;
        }
        const u32x4 kv = ld16(values + e.val_off + (int64_t)r * (bk / 2) + 16 * w);
        const uint32_t word = meta[e.meta_off + (int64_t)r * wpr + w];
        uint32_t out[8];
#pragma unroll
        for (int g = 0; g < 8; ++g) {   // group g: kept bytes 2g, 2g+1 of the chunk
            const uint32_t pair = (kv[g / 2] >> (16 * (g & 1))) & 0xFFFFu;
            const uint32_t code = (word >> (4 * g)) & 0xFu, i0 = code & 3u, i1 = code >> 2;
            out[g] = ((pair & 0xFFu) << (8 * i0)) | ((pair >> 8) << (8 * i1));
        }
        st16(dst, u32x4{out[0], out[1], out[2], out[3]});
        st16(dst + 16, u32x4{out[4], out[5], out[6], out[7]});
    }
}

}  // namespace

hipError_t launch_pack(const hts_desc& d, const hts_tile* index, const uint16_t* W, int64_t ldw,
                       const float* col_scale, uint16_t* values, uint32_t* meta, hipStream_t s) {
    const int64_t Tk = d.K / d.bk, T = (d.N / d.bn) * Tk;
    if (d.dtype == HTS_FP8_E4M3)
        pack8_kernel<false><<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, reinterpret_cast<const uint8_t*>(W), ldw, col_scale, nullptr, 0, nullptr,
            reinterpret_cast<uint8_t*>(values), meta);
    else if (d.dtype == HTS_BF16)
        pack_kernel<BF16T, false><<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, W, ldw, col_scale, nullptr, 0, nullptr, values, meta);
    else
        pack_kernel<F16T, false><<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, W, ldw, col_scale, nullptr, 0, nullptr, values, meta);
    return hipGetLastError();
}

hipError_t launch_pack_masked(const hts_desc& d, const hts_tile* index, const uint16_t* W, int64_t ldw,
                              const uint8_t* mask, int64_t ldm, uint32_t* malformed, uint16_t* values,
                              uint32_t* meta, hipStream_t s) {
    const int64_t Tk = d.K / d.bk, T = (d.N / d.bn) * Tk;
    if (malformed) zero_counter<<<dim3(1), dim3(1), 0, s>>>(malformed);   // a kernel, not a memset node
    if (d.dtype == HTS_FP8_E4M3)
        pack8_kernel<true><<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, reinterpret_cast<const uint8_t*>(W), ldw, nullptr, mask, ldm, malformed,
            reinterpret_cast<uint8_t*>(values), meta);
    else if (d.dtype == HTS_BF16)
        pack_kernel<BF16T, true><<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, W, ldw, nullptr, mask, ldm, malformed, values, meta);
    else
        pack_kernel<F16T, true><<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, W, ldw, nullptr, mask, ldm, malformed, values, meta);
    return hipGetLastError();
}

hipError_t launch_unpack(const hts_desc& d, const hts_tile* index, const uint16_t* values,
                         const uint32_t* meta, uint16_t* W_out, int64_t ldw, hipStream_t s) {
    const int64_t Tk = d.K / d.bk, T = (d.N / d.bn) * Tk;
    if (d.dtype == HTS_FP8_E4M3) {
        unpack8_kernel<<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(
            index, Tk, d.bn, d.bk, reinterpret_cast<const uint8_t*>(values), meta, reinterpret_cast<uint8_t*>(W_out),
            ldw);
        return hipGetLastError();
    }
    unpack_kernel<<<dim3((unsigned)T), dim3(kPackThreads), 0, s>>>(index, Tk, d.bn, d.bk, values, meta,
                                                                   W_out, ldw);
    return hipGetLastError();
}

}  // namespace hts
