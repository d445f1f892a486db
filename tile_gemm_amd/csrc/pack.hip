// Pack / unpack of a tile-level hybrid (dense / 2:4) weight on gfx950.
//
// One workgroup per tile (page "PATCH: Learnable Tile-level Hybrid Sparsity for
// LLMs", section 2: the dense / 2:4 decision is made per tile).  Each thread
// handles one 16-byte chunk of a tile row per step: a raw copy (dense tile) or
// two (four for 8-bit weights) 2-of-4 selections producing the kept values and
// their codes (2:4 tile).  The pass is bound by HBM bandwidth: it reads W once
// and writes the packed bytes once.
#include "device_common.h"
#include "hts_internal.h"

namespace hts {
namespace {

constexpr int kPackThreads = 256;
constexpr int kInFlight = 4;   // 16-byte chunks a pack thread loads before it uses any

// Storage order inside a tile: rows cut into 16-row panels (tiles have 32, 64 or 128 rows) and
// 16-byte chunks; in a panel the chunks are stored column by column, the panel's rows consecutive
// within a chunk column, so one matrix-core operand (a chunk of 16 consecutive rows, for four
// consecutive chunk columns) is one contiguous kilobyte.  Offset, in elements, of chunk c of row
// r of a stored block with w elements per row and ce elements per chunk:
__device__ __forceinline__ int64_t stored_chunk(int r, int c, int w, int ce) {
    return (int64_t)(r >> 4) * 16 * w + ((int64_t)c * 16 + (r & 15)) * ce;
}

// Work item -> (row, chunk) of a tile: 8 consecutive rows fastest, then the chunks of the row,
// then the next 8 rows -- a wave reads whole 128-byte lines of W and writes whole 128-byte runs.
__device__ __forceinline__ void item_rc(int it, int cpr, int& r, int& c) {
    const int rest = it >> 3;
    c = rest % cpr;
    r = 8 * (rest / cpr) + (it & 7);
}

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
//
// Work split: a thread takes one 16-byte chunk of a tile row per step (8 weights = two groups),
// consecutive lanes on consecutive chunks, so every load and store of a wave covers whole cache
// lines.  A 2:4 chunk becomes 8 stored bytes and one metadata byte: the codes of its two groups
// (group g's nibble is bits 4(g%8).. of word g/8 of the row, so groups 2c and 2c+1 are byte c).
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
    const int cpr = bk / 8;                        // 16-byte chunks per tile row
    const int items = bn * cpr;
    uint8_t* mbytes = reinterpret_cast<uint8_t*>(meta + e.meta_off);
    // kInFlight chunks per thread are loaded before any is used (guarded: small tiles have fewer
    // chunks than kInFlight x 256)
    for (int base = threadIdx.x; base < items; base += kInFlight * kPackThreads) {
        u32x4 qs[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            int r, c;
            item_rc(it, cpr, r, c);
            if (it < items) qs[j] = ld16(W + (tn * bn + r) * ldw + tk * bk + 8 * c);
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            if (it >= items) break;
            int r, c;
            item_rc(it, cpr, r, c);
            const int64_t k0 = tk * bk + 8 * c;
            const u32x4 q = qs[j];
            if (e.type == HTS_TILE_DENSE) {
                st16(values + e.val_off + stored_chunk(r, c, bk, 8), q);
                continue;
            }
            uint2 mk = {0u, 0u};   // mask bytes of the chunk's 8 weights
            if (MASKED) mk = *reinterpret_cast<const uint2*>(mask + (tn * bn + r) * ldm + k0);
            uint32_t kept[2];      // kept pair of each group, two 16-bit values per word
            uint32_t code = 0;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const uint32_t d0 = q[2 * g], d1 = q[2 * g + 1];
                const uint32_t b[4] = {d0 & 0xFFFFu, d0 >> 16, d1 & 0xFFFFu, d1 >> 16};
                float s[4];
                if (MASKED) {
                    const uint32_t mw = g ? mk.y : mk.x;      // mask bytes of the group's four weights
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
                code |= (i0 | (i1 << 2)) << (4 * g);
            }
            // the 4 kept values are half (c % 2) of stored chunk c / 2
            *reinterpret_cast<uint2*>(values + e.val_off + stored_chunk(r, c >> 1, bk / 2, 8) + 4 * (c & 1)) =
                uint2{kept[0], kept[1]};
            mbytes[(int64_t)r * (bk / 8) + c] = (uint8_t)code;
        }
    }
    if (MASKED && malformed && bad) atomicAdd(malformed, bad);
}

// The same pass for 8-bit E4M3 weights: a 16-byte chunk is 16 weights (four groups); a 2:4 chunk
// becomes 8 kept bytes and 16 bits of codes (metadata bytes 2c, 2c+1 of the row).  The score is
// |w| decoded exactly (times the column scale when given).
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
    const int cpr = bk / 16;
    const int items = bn * cpr;
    uint16_t* mhalves = reinterpret_cast<uint16_t*>(meta + e.meta_off);
    for (int base = threadIdx.x; base < items; base += kInFlight * kPackThreads) {
        u32x4 qs[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            int r, c;
            item_rc(it, cpr, r, c);
            if (it < items) qs[j] = ld16(W + (tn * bn + r) * ldw + tk * bk + 16 * c);
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            if (it >= items) break;
            int r, c;
            item_rc(it, cpr, r, c);
            const int64_t k0 = tk * bk + 16 * c;
            const u32x4 q = qs[j];
            if (e.type == HTS_TILE_DENSE) {
                st16(values + e.val_off + stored_chunk(r, c, bk, 16), q);
                continue;
            }
            u32x4 mk = {0u, 0u, 0u, 0u};
            if (MASKED) mk = *reinterpret_cast<const u32x4*>(mask + (tn * bn + r) * ldm + k0);
            uint32_t kept[4];   // kept pair of group g: low byte = lower index
            uint32_t code = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const uint32_t d = q[g];
                const uint32_t b[4] = {d & 0xFFu, (d >> 8) & 0xFFu, (d >> 16) & 0xFFu, d >> 24};
                float sc[4];
                if (MASKED) {
                    const uint32_t mw = mk[g];
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
                code |= (i0 | (i1 << 2)) << (4 * g);
            }
            *reinterpret_cast<uint2*>(values + e.val_off + stored_chunk(r, c >> 1, bk / 2, 16) + 8 * (c & 1)) =
                uint2{kept[0] | (kept[1] << 16), kept[2] | (kept[3] << 16)};
            mhalves[(int64_t)r * (bk / 16) + c] = (uint16_t)code;
        }
    }
    if (MASKED && malformed && bad) atomicAdd(malformed, bad);
}

__global__ void zero_counter(uint32_t* c) { *c = 0u; }

// Inverse passes, one 16-byte output chunk per thread and step (as the packs above).
__global__ __launch_bounds__(kPackThreads) void unpack_kernel(
    const hts_tile* __restrict__ index, int64_t Tk, int bn, int bk,
    const uint16_t* __restrict__ values, const uint32_t* __restrict__ meta,
    uint16_t* __restrict__ W, int64_t ldw) {
    const int64_t t = blockIdx.x;
    const hts_tile e = index[t];
    const int64_t tn = t / Tk, tk = t % Tk;
    const int cpr = bk / 8;
    const int items = bn * cpr;
    const uint8_t* mbytes = reinterpret_cast<const uint8_t*>(meta + e.meta_off);
    const bool dense = e.type == HTS_TILE_DENSE;
    for (int base = threadIdx.x; base < items; base += kInFlight * kPackThreads) {
        u32x4 q[kInFlight];        // dense: the chunk; 2:4: stored values in .x, .y and the code byte in .z
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            if (it >= items) break;
            int r, c;
            item_rc(it, cpr, r, c);
            if (dense) {
                q[j] = ld16(values + e.val_off + stored_chunk(r, c, bk, 8));
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(values + e.val_off + stored_chunk(r, c >> 1, bk / 2, 8) +
                                                                4 * (c & 1));
                q[j] = u32x4{v.x, v.y, mbytes[(int64_t)r * (bk / 8) + c], 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            if (it >= items) break;
            int r, c;
            item_rc(it, cpr, r, c);
            uint16_t* dst = W + (tn * bn + r) * ldw + tk * bk + 8 * c;
            st16(dst, dense ? q[j] : expand_two_groups(uint2{q[j][0], q[j][1]}, q[j][2]));
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
    const int cpr = bk / 16;
    const int items = bn * cpr;
    const uint16_t* mhalves = reinterpret_cast<const uint16_t*>(meta + e.meta_off);
    const bool dense = e.type == HTS_TILE_DENSE;
    for (int base = threadIdx.x; base < items; base += kInFlight * kPackThreads) {
        u32x4 q[kInFlight];        // dense: the chunk; 2:4: kept bytes in .x, .y and the codes in .z
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            if (it >= items) break;
            int r, c;
            item_rc(it, cpr, r, c);
            if (dense) {
                q[j] = ld16(values + e.val_off + stored_chunk(r, c, bk, 16));
            } else {
                const uint2 kv = *reinterpret_cast<const uint2*>(values + e.val_off + stored_chunk(r, c >> 1, bk / 2, 16) +
                                                                 8 * (c & 1));
                q[j] = u32x4{kv.x, kv.y, mhalves[(int64_t)r * (bk / 16) + c], 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int it = base + j * kPackThreads;
            if (it >= items) break;
            int r, c;
            item_rc(it, cpr, r, c);
            uint8_t* dst = W + (tn * bn + r) * ldw + tk * bk + 16 * c;
            if (dense) {
                st16(dst, q[j]);
                continue;
            }
            uint32_t out[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {   // group g: kept bytes 2g, 2g+1 of the chunk's 8
                const uint32_t pair = ((g < 2 ? q[j][0] : q[j][1]) >> (16 * (g & 1))) & 0xFFFFu;
                const uint32_t code = (q[j][2] >> (4 * g)) & 0xFu, i0 = code & 3u, i1 = code >> 2;
                out[g] = ((pair & 0xFFu) << (8 * i0)) | ((pair >> 8) << (8 * i1));
            }
            st16(dst, u32x4{out[0], out[1], out[2], out[3]});
        }
    }
}

// Debug check of a tile index in device memory (HTS_DEBUG=1): record t must have type 0 or 1, a
// zero reserved word, and offsets equal to those of record t-1 plus that tile's stored size
// (record 0 at offset 0), i.e. the prefix sums the plan wrote.  One thread per record; counts the
// bad records, keeps the first, and reports where the last tile's values and codes end.
__global__ __launch_bounds__(256) void index_check_kernel(const hts_tile* __restrict__ index, int64_t T,
                                                          uint32_t dense, uint32_t sparse, uint32_t mwords,
                                                          IndexCheck* out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const hts_tile e = index[t];
    bool ok = e.type <= 1u && e.reserved == 0u;
    if (t == 0) {
        ok = ok && e.val_off == 0u && e.meta_off == 0u;
    } else {
        const hts_tile p = index[t - 1];
        ok = ok && p.type <= 1u && e.val_off == p.val_off + (p.type ? sparse : dense) &&
             e.meta_off == p.meta_off + (p.type ? mwords : 0u);
    }
    if (!ok) {
        atomicAdd(&out->bad, 1u);
        atomicMin(&out->first_bad, (uint32_t)t);
    }
    if (t == T - 1 && e.type <= 1u) {
        out->values_end = (uint64_t)e.val_off + (e.type ? sparse : dense);
        out->meta_end = (uint64_t)e.meta_off + (e.type ? mwords : 0u);
    }
}

}  // namespace

hipError_t launch_index_check(const hts_desc& d, const hts_tile* index, IndexCheck* out, hipStream_t s) {
    const int64_t T = (d.N / d.bn) * (d.K / d.bk);
    const uint32_t dense = (uint32_t)(d.bn * d.bk);
    index_check_kernel<<<dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s>>>(index, T, dense, dense / 2, dense / 32,
                                                                               out);
    return hipGetLastError();
}

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
