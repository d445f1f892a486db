// Hybrid tile-sparse product for larger M: the matrix-core-bound tiled path.
//
// A workgroup of 4 waves owns a 128 (N) x 128 (M) block of Y^T = W . X^T and
// walks K in 64-wide slices.  Each slice of W (two 64-row halves, each half from
// one tile: dense, or 2:4 stored values + codes) and of X is staged through LDS,
// double-buffered, with XOR-swizzled 16-byte chunks so that the fragment reads
// of the matrix-core operands are free of bank conflicts.  Wave (wn, wm)
// computes rows 64*wn.. (one half) x columns 64*wm.. as 4 x 4 blocks of 16x16,
// feeding every slice to the matrix cores by its tile type: dense -> 16x16x32
// MFMA, 2:4 -> 16x16x64 SMFMAC (or expansion to dense MFMA), into the same fp32
// accumulators (page "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs",
// section 2, inference and deployment; 128 x 128 execution tiles, section 2 and
// the tile-size ablation of section 4).
//
// Workgroups are numbered so that each XCD (own L2) receives a contiguous range
// of output blocks, walked in groups of 8 N-blocks with M fastest, so the
// blocks running together on one XCD share their W and X slices in its L2.
#include "gemm_common.h"

namespace hts {
namespace {

constexpr int kBN = 128, kBM = 128, kKS = 64, kThreads = 256;
constexpr int kXBytes = kBM * kKS * 2;              // 16 KiB: X slice, 128 rows x 128 B
constexpr int kHalfBytes = 64 * kKS * 2;            // 8 KiB: one 64-row W half (dense)
constexpr int kMetaBytes = 2 * 64 * 8;              // two halves x 64 rows x 2 words
constexpr int kStageBytes = kXBytes + 2 * kHalfBytes + kMetaBytes;
constexpr int kGroupN = 8;

// byte offset of 16-byte chunk c of row r in a 128-byte-row buffer / 64-byte-row buffer
__device__ __forceinline__ int sw128(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int sw64(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 2) & 3)); }

struct HalfInfo {
    uint32_t type;          // HTS_TILE_DENSE / HTS_TILE_SPARSE24, or 2 = outside W
    const uint16_t* vals;   // first stored value of this slice for row 0 of the half
    int64_t rstride;        // elements between rows
    const uint32_t* meta;   // metadata words of this slice for row 0 (2:4 only)
    int64_t mstride;
};

template <int BK, bool HYB>
__device__ __forceinline__ HalfInfo half_info(const GemmArgs& a, int64_t n0, int hh, int64_t ks) {
    HalfInfo h;
    const int64_t nh = n0 + 64 * hh;
    h.meta = nullptr;
    h.mstride = 0;
    if (nh >= a.N) {
        h.type = 2;
        h.vals = nullptr;
        h.rstride = 0;
        return h;
    }
    if (!HYB) {
        h.type = HTS_TILE_DENSE;
        h.vals = a.W + nh * a.ldw + ks * kKS;
        h.rstride = a.ldw;
        return h;
    }
    const int64_t Tk = a.K / BK;
    const int64_t tn = nh / a.bn, r = nh - tn * a.bn;
    const int64_t tk = ks / (BK / kKS), s = ks % (BK / kKS);
    const hts_tile e = a.index[tn * Tk + tk];
    h.type = e.type;
    if (e.type == HTS_TILE_DENSE) {
        h.rstride = BK;
        h.vals = a.values + e.val_off + r * BK + s * kKS;
    } else {
        h.rstride = BK / 2;
        h.vals = a.values + e.val_off + r * (BK / 2) + s * (kKS / 2);
        h.mstride = BK / 32;
        h.meta = a.meta + e.meta_off + r * (BK / 32) + 2 * s;
    }
    return h;
}

struct Staging {
    u32x4 x[4];
    u32x4 w[2][2];
    uint2 m[2];
    uint32_t type[2];
};

template <int BK, bool HYB>
__device__ __forceinline__ void load_slice(Staging& S, const GemmArgs& a, int64_t n0, int64_t m0,
                                           int64_t ks, int tid) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int c = tid + kThreads * v, row = c >> 3, col = c & 7;
        const int64_t m = m0 + row;
        const u32x4 z = {0u, 0u, 0u, 0u};
        S.x[v] = (m < a.M) ? ld16(a.X + m * a.ldx + ks * kKS + 8 * col) : z;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const HalfInfo h = half_info<BK, HYB>(a, n0, hh, ks);
        S.type[hh] = h.type;
        if (h.type == HTS_TILE_DENSE) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int c = tid + kThreads * v, row = c >> 3, col = c & 7;
                S.w[hh][v] = ld16(h.vals + row * h.rstride + 8 * col);
            }
        } else if (h.type == HTS_TILE_SPARSE24) {
            const int row = tid >> 2, col = tid & 3;
            S.w[hh][0] = ld16(h.vals + row * h.rstride + 8 * col);
            if (tid < 64) S.m[hh] = *reinterpret_cast<const uint2*>(h.meta + tid * h.mstride);
        }
    }
}

__device__ __forceinline__ void store_slice(const Staging& S, uint8_t* stage, int tid) {
    uint8_t* xs = stage;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int c = tid + kThreads * v, row = c >> 3, col = c & 7;
        st16(xs + sw128(row, col), S.x[v]);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        uint8_t* ws = stage + kXBytes + hh * kHalfBytes;
        if (S.type[hh] == HTS_TILE_DENSE) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int c = tid + kThreads * v, row = c >> 3, col = c & 7;
                st16(ws + sw128(row, col), S.w[hh][v]);
            }
        } else if (S.type[hh] == HTS_TILE_SPARSE24) {
            const int row = tid >> 2, col = tid & 3;
            st16(ws + sw64(row, col), S.w[hh][0]);
            if (tid < 64)
                *reinterpret_cast<uint2*>(stage + kXBytes + 2 * kHalfBytes + hh * 512 + tid * 8) = S.m[hh];
        }
    }
}

template <typename T, int SP>
__device__ __forceinline__ void compute_slice(f32x4 (&acc)[4][4], const uint8_t* stage, uint32_t type,
                                              int wn, int wm, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const uint8_t* xs = stage;
    const uint8_t* ws = stage + kXBytes + wn * kHalfBytes;
    const uint32_t* ms = reinterpret_cast<const uint32_t*>(stage + kXBytes + 2 * kHalfBytes + wn * 512);
    if (type == HTS_TILE_DENSE || SP == SPARSE_DECOMPRESS) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int chunk = koff<SP>(u, g) / 8;
            u32x4 A[4], B[4];
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) B[bj] = ld16(xs + sw128(64 * wm + 16 * bj + i, chunk));
            if (type == HTS_TILE_DENSE) {
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) A[bi] = ld16(ws + sw128(16 * bi + i, chunk));
            } else {
                // expansion order: lane group g, substep u covers dense k [16g + 8u, +8) of the
                // slice = groups 4g + 2u, +1: stored bytes 16g + 8u, codes at bit 16g + 8u
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
                    const int row = 16 * bi + i;
                    const uint2 v = *reinterpret_cast<const uint2*>(ws + sw64(row, g) + 8 * u);
                    const uint32_t code = (ms[2 * row + (g >> 1)] >> (16 * (g & 1) + 8 * u)) & 0xFFu;
                    A[bi] = expand_two_groups(v, code);
                }
            }
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = mfma_dense<T>(A[bi], B[bj], acc[bi][bj]);
        }
    } else {
        u32x4 A[4], B0[4], B1[4];
        uint32_t idx[4];
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int row = 64 * wm + 16 * bj + i;
            B0[bj] = ld16(xs + sw128(row, g));
            B1[bj] = ld16(xs + sw128(row, 4 + g));
        }
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            const int row = 16 * bi + i;
            A[bi] = ld16(ws + sw64(row, g));
            idx[bi] = ms[2 * row + (g >> 1)] >> (16 * (g & 1));
        }
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                acc[bi][bj] = mfma_sparse<T, 0>(A[bi], B0[bj], B1[bj], idx[bi], acc[bi][bj]);
    }
}

template <typename T, int BK, bool HYB, int SP>
__global__ __launch_bounds__(kThreads) void gemm_prefill_kernel(const GemmArgs a, int NB, int MB) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2][kStageBytes];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;

    // block id -> output block: contiguous ranges per XCD, grouped along N, M fastest
    const int64_t total = (int64_t)NB * MB, L = blockIdx.x;
    const int64_t P = total / 8;
    const int64_t id = (L < 8 * P) ? (L % 8) * P + L / 8 : L;
    const int64_t gsz = (int64_t)kGroupN * MB;
    const int64_t grp = id / gsz, inb = id % gsz;
    const int64_t nb0 = grp * kGroupN;
    const int64_t gn = (NB - nb0 < kGroupN) ? (NB - nb0) : kGroupN;
    const int64_t nb = nb0 + inb % gn, mb = inb / gn;
    const int64_t n0 = nb * kBN, m0 = mb * kBM;

    f32x4 acc[4][4];
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[bi][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t S = a.K / kKS;
    Staging st;
    load_slice<BK, HYB>(st, a, n0, m0, 0, tid);
    store_slice(st, smem[0], tid);
    uint32_t cur_type[2] = {st.type[0], st.type[1]};
    __syncthreads();
    for (int64_t ks = 0; ks < S; ++ks) {
        const bool more = ks + 1 < S;
        if (more) load_slice<BK, HYB>(st, a, n0, m0, ks + 1, tid);
        const uint32_t ty = cur_type[wn];
        if (ty != 2) compute_slice<T, SP>(acc, smem[ks & 1], ty, wn, wm, lane);
        if (more) {
            store_slice(st, smem[(ks + 1) & 1], tid);
            cur_type[0] = st.type[0];
            cur_type[1] = st.type[1];
        }
        __syncthreads();
    }

    // epilogue: acc[bi][bj] lane (j + 16q) holds Y^T rows 4q..4q+3 of block bi, column j of block bj
    if (n0 + 64 * wn >= a.N) return;
    const int j = lane & 15, q = lane >> 4;
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const int64_t m = m0 + 64 * wm + 16 * bj + j;
        if (m >= a.M) continue;
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
            const int64_t n = n0 + 64 * wn + 16 * bi + 4 * q;
            store_y4(a.Y, m * a.ldy + n, a.y_dtype, acc[bi][bj]);
        }
    }
}

template <typename T, int BK, bool HYB>
hipError_t launch3(const GemmArgs& a, int sp, hipStream_t s) {
    const int NB = (int)((a.N + kBN - 1) / kBN), MB = (int)((a.M + kBM - 1) / kBM);
    const dim3 grid((unsigned)(NB * MB));
    if (sp == SPARSE_SMFMAC)
        gemm_prefill_kernel<T, BK, HYB, SPARSE_SMFMAC><<<grid, dim3(kThreads), 0, s>>>(a, NB, MB);
    else
        gemm_prefill_kernel<T, BK, HYB, SPARSE_DECOMPRESS><<<grid, dim3(kThreads), 0, s>>>(a, NB, MB);
    return hipGetLastError();
}

template <typename T>
hipError_t launch2(const GemmArgs& a, int sp, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128) return hyb ? launch3<T, 128, true>(a, sp, s) : launch3<T, 128, false>(a, sp, s);
    return hyb ? launch3<T, 64, true>(a, sp, s) : launch3<T, 64, false>(a, sp, s);
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, int sparse_path, hipStream_t s) {
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, sparse_path, s) : launch2<F16T>(a, sparse_path, s);
}

}  // namespace hts
