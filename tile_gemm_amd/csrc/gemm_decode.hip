// Hybrid tile-sparse product for small M (M <= 16): the HBM-streaming path.
//
// At decode-sized M the weight bytes are almost all of the traffic, so every
// weight byte is read once, straight from HBM into registers, with no LDS
// staging.  A workgroup owns a 16-row panel of W and KSPLIT waves; each wave
// walks its share of that panel's tile row (shares balanced by packed bytes,
// read from the tile index) and feeds each tile to the matrix cores by type:
// dense tiles -> 16x16x32 MFMA, 2:4 tiles -> 16x16x64 SMFMAC (or in-register
// expansion to dense MFMA), all into one fp32 accumulator (page "PATCH:
// Learnable Tile-level Hybrid Sparsity for LLMs", section 2, inference and
// deployment: sparse tiles on the sparse matrix cores, dense tiles on the dense
// ones).  The KSPLIT partial sums meet in LDS and are added in a fixed order.
//
// Registers per tile, lane L = i + 16g (weights: row i; X: row j = i):
//   dense substep u: weights W[i][koff(u,g) .. +8], X[j][koff(u,g) .. +8]
//   2:4 slice s   : the 8 stored values of row i for dense k in [64s+16g, +16)
//                   (stored offset 32s + 8g) and the 16-bit code half (g & 1)
//                   of metadata word 2s + g/2 of that row.
#include "gemm_common.h"

namespace hts {
namespace {

template <int BK>
struct TileRegs {
    u32x4 a[BK / 32];      // dense: BK/32 chunks; 2:4: BK/64 chunks
    uint32_t m[BK / 64];   // 2:4 metadata words, one per slice
    u32x4 x[BK / 32];      // X chunks
    uint32_t type;
};

template <typename T, int BK, bool HYB, int SP>
__device__ __forceinline__ void load_tile(TileRegs<BK>& R, const GemmArgs& a, int64_t t, int64_t tk,
                                          int64_t n0, int r0, int lane, bool xvalid,
                                          const uint16_t* xrow) {
    const int i = lane & 15, g = lane >> 4;
    uint32_t type = HTS_TILE_DENSE;
    const uint16_t* base;
    uint32_t moff = 0;
    if (HYB) {
        const hts_tile e = a.index[t];
        type = e.type;
        moff = e.meta_off;
        base = a.values + e.val_off + (int64_t)(r0 + i) * (type == HTS_TILE_DENSE ? BK : BK / 2);
    } else {
        base = a.W + (n0 + i) * a.ldw + tk * BK;
    }
    R.type = type;
    if (type == HTS_TILE_DENSE) {
#pragma unroll
        for (int u = 0; u < BK / 32; ++u) R.a[u] = ld16(base + koff<SP>(u, g));
    } else {
        const uint32_t* mrow = a.meta + moff + (int64_t)(r0 + i) * (BK / 32);
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) {
            R.a[s] = ld16(base + 32 * s + 8 * g);
            R.m[s] = mrow[2 * s + (g >> 1)];
        }
    }
#pragma unroll
    for (int u = 0; u < BK / 32; ++u) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        R.x[u] = xvalid ? ld16(xrow + tk * BK + koff<SP>(u, g)) : z;
    }
}

template <typename T, int BK, int SP>
__device__ __forceinline__ f32x4 mma_tile(const TileRegs<BK>& R, f32x4 acc, int lane) {
    const int g = lane >> 4;
    if (R.type == HTS_TILE_DENSE) {
#pragma unroll
        for (int u = 0; u < BK / 32; ++u) acc = mfma_dense<T>(R.a[u], R.x[u], acc);
    } else {
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) {
            const uint32_t code = R.m[s] >> (16 * (g & 1));
            if (SP == SPARSE_SMFMAC) {
                acc = mfma_sparse<T, 0>(R.a[s], cat8(R.x[2 * s], R.x[2 * s + 1]), code, acc);
            } else {
                const u32x4 v = R.a[s];
                acc = mfma_dense<T>(expand_two_groups(uint2{v[0], v[1]}, code & 0xFFu), R.x[2 * s], acc);
                acc = mfma_dense<T>(expand_two_groups(uint2{v[2], v[3]}, (code >> 8) & 0xFFu),
                                    R.x[2 * s + 1], acc);
            }
        }
    }
    return acc;
}

template <typename T, int BK, bool HYB, int SP, int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void gemm_decode_kernel(const GemmArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t tn = n0 / a.bn;
    const int r0 = (int)(n0 - tn * a.bn);
    const int64_t Tk = a.K / BK, t0 = tn * Tk;

    // This wave's tiles [kb, ke) of the tile row.
    int64_t kb, ke;
    if (HYB) {
        // balanced by packed size: tile tk goes to the wave whose byte range holds its start
        const hts_tile first = a.index[t0], last = a.index[t0 + Tk - 1];
        const uint64_t base = first.val_off;
        const uint64_t total = (uint64_t)last.val_off - base +
                               (last.type == HTS_TILE_DENSE ? (uint64_t)a.bn * BK : (uint64_t)a.bn * BK / 2);
        const uint64_t lo = total * wave / KSPLIT, hi = total * (wave + 1) / KSPLIT;
        int64_t clo = 0, chi = 0;
        for (int64_t x0 = 0; x0 < Tk; x0 += 64) {
            const int64_t x = x0 + lane;
            uint64_t rel = ~0ull;
            if (x < Tk) rel = (uint64_t)a.index[t0 + x].val_off - base;
            clo += __popcll(__ballot(rel < lo));
            chi += __popcll(__ballot(rel < hi));
        }
        kb = clo;
        ke = chi;
    } else {
        kb = Tk * wave / KSPLIT;
        ke = Tk * (wave + 1) / KSPLIT;
    }

    const int j = lane & 15;
    const bool xvalid = j < a.M;
    const uint16_t* xrow = a.X + (xvalid ? (int64_t)j * a.ldx : 0);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    TileRegs<BK> R0, R1;
    if (kb < ke) load_tile<T, BK, HYB, SP>(R0, a, t0 + kb, kb, n0, r0, lane, xvalid, xrow);
    for (int64_t tk = kb; tk < ke; tk += 2) {
        if (tk + 1 < ke) load_tile<T, BK, HYB, SP>(R1, a, t0 + tk + 1, tk + 1, n0, r0, lane, xvalid, xrow);
        acc = mma_tile<T, BK, SP>(R0, acc, lane);
        if (tk + 1 >= ke) break;
        if (tk + 2 < ke) load_tile<T, BK, HYB, SP>(R0, a, t0 + tk + 2, tk + 2, n0, r0, lane, xvalid, xrow);
        acc = mma_tile<T, BK, SP>(R1, acc, lane);
    }

    __shared__ f32x4 red[KSPLIT][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < 256) {
        // output (row rr of the panel, column m of Y^T): lane m + 16*(rr/4), component rr%4
        const int m = threadIdx.x >> 4, rr = threadIdx.x & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < KSPLIT; ++w) sum += red[w][m + 16 * (rr >> 2)][rr & 3];
        if (m < a.M) store_y1(a.Y, (int64_t)m * a.ldy + n0 + rr, a.y_dtype, sum);
    }
}

template <typename T, int BK, bool HYB, int SP>
hipError_t launch4(const GemmArgs& a, int ksplit, hipStream_t s) {
    const dim3 grid((unsigned)(a.N / 16));
    if (ksplit == 8)
        gemm_decode_kernel<T, BK, HYB, SP, 8><<<grid, dim3(512), 0, s>>>(a);
    else
        gemm_decode_kernel<T, BK, HYB, SP, 4><<<grid, dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, int BK, bool HYB>
hipError_t launch3(const GemmArgs& a, int ksplit, int sp, hipStream_t s) {
    return sp == SPARSE_SMFMAC ? launch4<T, BK, HYB, SPARSE_SMFMAC>(a, ksplit, s)
                               : launch4<T, BK, HYB, SPARSE_DECOMPRESS>(a, ksplit, s);
}

template <typename T>
hipError_t launch2(const GemmArgs& a, int ksplit, int sp, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128)
        return hyb ? launch3<T, 128, true>(a, ksplit, sp, s) : launch3<T, 128, false>(a, ksplit, sp, s);
    return hyb ? launch3<T, 64, true>(a, ksplit, sp, s) : launch3<T, 64, false>(a, ksplit, sp, s);
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs& a, int ksplit, int sparse_path, hipStream_t s) {
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, ksplit, sparse_path, s)
                               : launch2<F16T>(a, ksplit, sparse_path, s);
}

}  // namespace hts
