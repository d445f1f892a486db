// Hybrid tile-sparse product for small M (M <= 16): the HBM-streaming path.
//
// At decode-sized M the weight bytes are almost all of the traffic, so every
// weight byte is read once, straight from HBM into registers, with no LDS
// staging.  A workgroup owns a 16-row panel of W and KS waves; wave w walks the
// tile columns [Tk*w/KS, Tk*(w+1)/KS) of the panel's tile row and feeds each tile
// to the matrix cores by its type: dense tiles -> 16x16x32 MFMA, 2:4 tiles ->
// 16x16x64 SMFMAC (or in-register expansion to dense MFMA), all into one fp32
// accumulator (page "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs",
// section 2, inference and deployment: sparse tiles on the sparse matrix cores,
// dense tiles on the dense ones).  The KS partial sums meet in LDS and are added
// in a fixed order, so results do not depend on timing.
//
// Memory-level parallelism: a wave takes its tiles NT at a time and issues every
// load of the NT tiles (weights, 2:4 codes and X) before the first use of any of
// them, so each wave keeps NT tiles of HBM reads in flight; branch-free X loads
// (rows past M repeat row M-1, whose output columns are never stored) keep the
// compiler from inserting early waits.  Workgroups are dealt to the 8 XCDs round
// robin by the hardware; the panel order below gives each XCD one contiguous run
// of panels, so each XCD streams whole tiles rather than scattered 4 KB slices.
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
};

template <typename T, int BK, bool HYB, int SP>
__device__ __forceinline__ uint32_t load_tile(TileRegs<BK>& R, const GemmArgs& a, int64_t t0, int tk,
                                              int64_t n0, int r0, int lane, const uint16_t* xrow) {
    const int i = lane & 15, g = lane >> 4;
    uint32_t type = HTS_TILE_DENSE;
    const uint16_t* base;
    uint32_t moff = 0;
    if (HYB) {
        const hts_tile e = a.index[t0 + tk];   // uniform: scalar load
        type = e.type;
        moff = e.meta_off;
        base = a.values + e.val_off + (int64_t)(r0 + i) * (type == HTS_TILE_DENSE ? BK : BK / 2);
    } else {
        base = a.W + (n0 + i) * a.ldw + (int64_t)tk * BK;
    }
    if (type == HTS_TILE_DENSE) {
#pragma unroll
        for (int u = 0; u < BK / 32; ++u) R.a[u] = ld16(base + koff<SP>(u, g));
    } else {
        const uint32_t* mrow = a.meta + moff + (int64_t)(r0 + i) * (BK / 32);
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) R.a[s] = ld16(base + 32 * s + 8 * g);
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) R.m[s] = mrow[2 * s + (g >> 1)];
    }
#pragma unroll
    for (int u = 0; u < BK / 32; ++u) R.x[u] = ld16(xrow + (int64_t)tk * BK + koff<SP>(u, g));
    return type;
}

template <typename T, int BK, int SP>
__device__ __forceinline__ f32x4 mma_tile(const TileRegs<BK>& R, uint32_t type, f32x4 acc, int lane) {
    const int g = lane >> 4;
    if (type == HTS_TILE_DENSE) {
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

template <typename T, int BK, bool HYB, int SP, int KS, int NT>
__global__ __launch_bounds__(64 * KS) void gemm_decode_kernel(const GemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD x (= blockIdx % 8) takes panels [x*q + min(x, r), ...) in order
    const uint32_t P = gridDim.x, b = blockIdx.x, x = b & 7u, q = P >> 3, r = P & 7u;
    const int64_t n0 = (int64_t)(x * q + (x < r ? x : r) + (b >> 3)) * 16;
    const int64_t tn = n0 / a.bn;
    const int r0 = (int)(n0 - tn * a.bn);
    const int Tk = (int)(a.K / BK);
    const int64_t t0 = tn * Tk;
    const int kb = Tk * wave / KS, ke = Tk * (wave + 1) / KS;

    const int i = lane & 15;
    const int64_t j = i < a.M ? i : a.M - 1;
    const uint16_t* xrow = a.X + j * a.ldx;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int t = kb; t < ke; t += NT) {
        TileRegs<BK> R[NT];
        uint32_t type[NT];
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) type[s] = load_tile<T, BK, HYB, SP>(R[s], a, t0, t + s, n0, r0, lane, xrow);
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) acc = mma_tile<T, BK, SP>(R[s], type[s], acc, lane);
    }

    __shared__ f32x4 red[KS][64];
    red[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x < 256) {
        // output (row rr of the panel, column m of Y^T): lane m + 16*(rr/4), component rr%4
        const int m = threadIdx.x >> 4, rr = threadIdx.x & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < KS; ++w) sum += red[w][m + 16 * (rr >> 2)][rr & 3];
        if (m < a.M) store_y1(a.Y, (int64_t)m * a.ldy + n0 + rr, a.y_dtype, sum);
    }
}

template <typename T, int BK, bool HYB, int SP, int KS>
hipError_t launch5(const GemmArgs& a, int nt, hipStream_t s) {
    const dim3 grid((unsigned)(a.N / 16)), block(64 * KS);
    // nt counts 128-wide tile columns; a 64-wide tile is half as many bytes.  With 16 waves
    // (at most 128 registers per lane) only the 2-column batch fits without spills.
    if constexpr (KS < 16) {
        if (nt >= 4) {
            gemm_decode_kernel<T, BK, HYB, SP, KS, 4 * 128 / BK><<<grid, block, 0, s>>>(a);
            return hipGetLastError();
        }
    }
    gemm_decode_kernel<T, BK, HYB, SP, KS, 2 * 128 / BK><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

template <typename T, int BK, bool HYB, int SP>
hipError_t launch4(const GemmArgs& a, int ksplit, int nt, hipStream_t s) {
    if (ksplit >= 16) return launch5<T, BK, HYB, SP, 16>(a, nt, s);
    if (ksplit >= 8) return launch5<T, BK, HYB, SP, 8>(a, nt, s);
    return launch5<T, BK, HYB, SP, 4>(a, nt, s);
}

template <typename T, int BK, bool HYB>
hipError_t launch3(const GemmArgs& a, int ksplit, int nt, int sp, hipStream_t s) {
    return sp == SPARSE_SMFMAC ? launch4<T, BK, HYB, SPARSE_SMFMAC>(a, ksplit, nt, s)
                               : launch4<T, BK, HYB, SPARSE_DECOMPRESS>(a, ksplit, nt, s);
}

template <typename T>
hipError_t launch2(const GemmArgs& a, int ksplit, int nt, int sp, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128)
        return hyb ? launch3<T, 128, true>(a, ksplit, nt, sp, s) : launch3<T, 128, false>(a, ksplit, nt, sp, s);
    return hyb ? launch3<T, 64, true>(a, ksplit, nt, sp, s) : launch3<T, 64, false>(a, ksplit, nt, sp, s);
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs& a, int ksplit, int nt, int sparse_path, hipStream_t s) {
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, ksplit, nt, sparse_path, s)
                               : launch2<F16T>(a, ksplit, nt, sparse_path, s);
}

}  // namespace hts
