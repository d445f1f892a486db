// Hybrid tile-sparse product for larger M: the matrix-core-bound tiled path.
//
// A workgroup of 4 waves (2 x 2) owns a BN (weight rows) x BM (X rows) block
// of Y^T = W . X^T and walks K in 64-wide slices.  Each slice of X and of the
// BN weight rows -- in groups of 64 rows, each group from one tile: dense
// values, or 2:4 stored values + 2-bit codes -- is copied from global memory
// straight into LDS (gfx950 global_load_lds_dwordx4: no register staging),
// double-buffered, into XOR-swizzled 16-byte chunks so the fragment reads of
// the matrix-core operands are free of bank conflicts.  Wave (wn, wm) computes
// BN/2 x BM/2 as 16x16 blocks; each 64-row group of a slice is fed to the
// matrix cores by its tile type -- dense: 16x16x32 MFMA, 2:4: 16x16x64 SMFMAC
// (or in-register expansion to dense MFMA) -- into the same fp32 accumulators
// (page "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", section 2,
// inference and deployment: 2:4 tiles on the sparse matrix cores, dense tiles
// on the dense ones; execution tiles of 128 x 128 and larger, sections 2 and 4).
//
// The tile index of the workgroup's tile rows is read into LDS once, so no
// weight load waits on an index load.  Workgroups are numbered so that each XCD
// (own L2) receives a contiguous range of output blocks, walked in groups of 8
// N-blocks with M fastest: blocks running together on one XCD share their W and
// X slices in its L2.
#include "gemm_common.h"

namespace hts {
namespace {

typedef __attribute__((address_space(3))) void lds_t;

constexpr int kKS = 64;                 // K elements per slice
constexpr int kThreads = 256;
constexpr int kGroupBytes = 64 * 128;   // one 64-row weight group, dense (2:4 uses half)
constexpr int kMetaGroupBytes = 64 * 8; // codes of one 64-row group for one slice
constexpr int kMaxTileCols = 256;       // K/bk limit: the tile list of a tile row is kept in LDS
constexpr int kGroupN = 8;

// LDS image of one stage: X slice (BM rows x 128 B), BN/64 weight groups, their codes.
template <int BN, int BM, int NSTAGE>
struct Layout {
    static constexpr int NG = BN / 64;
    static constexpr int WOFF = BM * 128;
    static constexpr int MOFF = WOFF + NG * kGroupBytes;
    static constexpr int STAGE = MOFF + NG * kMetaGroupBytes;
    static constexpr int SINK = NSTAGE * STAGE;              // target of the padding copies
    static constexpr int LIST = SINK + 1024;                 // ordered tile list: {val_off, meta_off}
    static constexpr int LCOL = LIST + kMaxTileCols * 8;     // ... and the tile column of each entry
    static constexpr int WCNT = LCOL + kMaxTileCols * 2;     // per-wave counts while ordering
    static constexpr int TOTAL = WCNT + 64;
};

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_t*)lds, 4, 0, 0);
}

// Everything the copy jobs need, fixed for the whole K loop.  A job moves 1 KiB (64
// lanes x 16 B) into contiguous LDS; each lane picks the global chunk whose swizzled
// LDS position is its slot.
template <int BK, bool HYB, int BN, int BM>
struct Ctx {
    static constexpr int NG = BN / 64;
    const uint16_t* values;
    const uint32_t* meta;
    const uint16_t* W;          // row-major weight (dense product), row n0
    int64_t ldw;
    int64_t N, n0;
    int r0;                     // first row of the block inside its tile (0 when BN == bn)
    int wave;
    int n_dense;                // dense tiles of the list (they come first)
    const uint2* list;          // {val_off, meta_off} of the tile row's tiles in list order
    int Tk;
    const uint16_t* xsrc[BM / 32];
    int d_row[2], d_col[2];     // dense group job rows / chunks (128 B rows)
    int s_row, s_col;           // 2:4 group job (64 B rows)
    int m_row, m_w;             // 2:4 codes job (one word per lane)
    __device__ __forceinline__ bool gvalid(int gi) const { return n0 + 64 * gi < N; }
};

// Issue the copies of slice ks into one LDS stage.  Every wave issues the same number of
// copy instructions for every slice, BM/32 + 2 * BN/64, whatever the tile type (a 2:4 group's
// codes need two 256-byte copies; waves 2 and 3 repeat them into a sink), so the wait for
// one slice is a fixed count of outstanding copies.
template <int BK, bool HYB, int BN, int BM, int NSTAGE>
__device__ __forceinline__ void issue_slice(const Ctx<BK, HYB, BN, BM>& C, int ks, uint8_t* stage, uint8_t* sink) {
    using Lo = Layout<BN, BM, NSTAGE>;
    constexpr int SPT = BK / kKS;
    const int p = ks / SPT, s = ks % SPT;     // list position, slice of the tile
    // read the list entry before any copy is issued: an LDS read after a copy into LDS makes
    // the compiler wait for every copy in flight
    uint32_t voff = 0, moff = 0;
    if (HYB) {
        const uint2 e = C.list[p];            // every group of the block is in the same tile
        voff = __builtin_amdgcn_readfirstlane(e.x);
        moff = __builtin_amdgcn_readfirstlane(e.y);
    }
#pragma unroll
    for (int v = 0; v < BM / 32; ++v) {
        // X columns of list position p: the tile column stored in the list entry (HYB), or p itself
        dma16(C.xsrc[v], stage + 1024 * (C.wave + 4 * v));
    }
    const bool dense = !HYB || p < C.n_dense;
#pragma unroll
    for (int gi = 0; gi < Lo::NG; ++gi) {
        if (!C.gvalid(gi)) {                    // rows past N: keep the copy count, land in the sink
            dma16(C.xsrc[0], sink);
            dma16(C.xsrc[0], sink);
            continue;
        }
        uint8_t* ws = stage + Lo::WOFF + gi * kGroupBytes;
        if (!HYB) {
            const uint16_t* base = C.W + 64 * gi * C.ldw + ks * kKS;
#pragma unroll
            for (int v = 0; v < 2; ++v)
                dma16(base + (int64_t)C.d_row[v] * C.ldw + 8 * C.d_col[v], ws + 1024 * (C.wave + 4 * v));
            continue;
        }
        const int r = C.r0 + 64 * gi;
        if (dense) {
            const uint16_t* base = C.values + voff + r * BK + s * kKS;
#pragma unroll
            for (int v = 0; v < 2; ++v)
                dma16(base + C.d_row[v] * BK + 8 * C.d_col[v], ws + 1024 * (C.wave + 4 * v));
        } else {
            const uint16_t* base = C.values + voff + r * (BK / 2) + s * (kKS / 2);
            dma16(base + C.s_row * (BK / 2) + 8 * C.s_col, ws + 1024 * C.wave);
            dma4(C.meta + moff + r * (BK / 32) + 2 * s + C.m_row * (BK / 32) + C.m_w,
                 C.wave < 2 ? stage + Lo::MOFF + gi * kMetaGroupBytes + 256 * C.wave : sink);
        }
    }
}

// X fragments of one slice for this wave: chunks c0 (low half) and c1 (high half) of each
// column block.  Rows 16b + i share the swizzle of row i.
template <int SP, int NBJ>
__device__ __forceinline__ void load_x(u32x8 (&Bx)[NBJ], const uint8_t* xs, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int c0 = (SP == SPARSE_SMFMAC) ? g : 2 * g;
    const int c1 = (SP == SPARSE_SMFMAC) ? 4 + g : 2 * g + 1;
    const int x0 = i * 128 + 16 * (c0 ^ ((i >> 1) & 7));
    const int x1 = i * 128 + 16 * (c1 ^ ((i >> 1) & 7));
#pragma unroll
    for (int bj = 0; bj < NBJ; ++bj) Bx[bj] = cat8(ld16(xs + bj * 2048 + x0), ld16(xs + bj * 2048 + x1));
}

template <typename T, int SP, int NBJ>
__device__ __forceinline__ void compute_dense(f32x4 (&acc)[4][NBJ], const uint8_t* xs, const uint8_t* ws, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int c0 = (SP == SPARSE_SMFMAC) ? g : 2 * g;
    const int c1 = (SP == SPARSE_SMFMAC) ? 4 + g : 2 * g + 1;
    const int a0 = i * 128 + 16 * (c0 ^ ((i >> 1) & 7));
    const int a1 = i * 128 + 16 * (c1 ^ ((i >> 1) & 7));
    u32x8 Bx[NBJ];
    load_x<SP, NBJ>(Bx, xs, lane);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        u32x4 A[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) A[b] = ld16(ws + b * 2048 + (u ? a1 : a0));
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int bj = 0; bj < NBJ; ++bj)
                acc[b][bj] = mfma_dense<T>(A[b], u ? hi4(Bx[bj]) : lo4(Bx[bj]), acc[b][bj]);
    }
}

template <typename T, int SP, int NBJ>
__device__ __forceinline__ void compute_sparse(f32x4 (&acc)[4][NBJ], const uint8_t* xs, const uint8_t* ws,
                                               const uint32_t* ms, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int s0 = i * 64 + 16 * (g ^ ((i >> 2) & 3));
    u32x8 Bx[NBJ];
    load_x<SP, NBJ>(Bx, xs, lane);
    if (SP == SPARSE_SMFMAC) {
        u32x4 A[4];
        uint32_t idx[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            A[b] = ld16(ws + b * 1024 + s0);
            idx[b] = ms[2 * (16 * b + i) + (g >> 1)] >> (16 * (g & 1));
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int bj = 0; bj < NBJ; ++bj) acc[b][bj] = mfma_sparse<T, 0>(A[b], Bx[bj], idx[b], acc[b][bj]);
    } else {
        // expansion order: lane group g, substep u covers dense k [16g + 8u, +8) of the slice =
        // groups 4g + 2u, +1: stored bytes 16g + 8u of the row, codes at bit 16g + 8u
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            u32x4 A[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint2 v = *reinterpret_cast<const uint2*>(ws + b * 1024 + s0 + 8 * u);
                const uint32_t code = (ms[2 * (16 * b + i) + (g >> 1)] >> (16 * (g & 1) + 8 * u)) & 0xFFu;
                A[b] = expand_two_groups(v, code);
            }
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int bj = 0; bj < NBJ; ++bj)
                    acc[b][bj] = mfma_dense<T>(A[b], u ? hi4(Bx[bj]) : lo4(Bx[bj]), acc[b][bj]);
        }
    }
}

// One workgroup = one tile row (BN = bn) x BM rows of X.  Waves: BN/64 along N (one
// 64-row group each) x the rest along M.  The tile row's tiles are walked as an ordered
// list -- all dense tiles, then all 2:4 tiles -- so each half of the K loop runs one
// instruction kind with no branch on the tile type (the sum does not depend on the order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt with vmcnt = N (low 4 bits and bits 14..15), expcnt and lgkmcnt left at their maxima
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T, int BK, bool HYB, int SP, int BN, int BM, int NSTAGE, bool ROT = false>
__global__ __launch_bounds__(kThreads) void gemm_prefill_kernel(const GemmArgs a, int NB, int MB) {
    using Lo = Layout<BN, BM, NSTAGE>;
    constexpr int NG = BN / 64, WM = 4 / NG, WTM = BM / WM, NBJ = WTM / 16, SPT = BK / kKS;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % NG, wm = wave / NG;

    // block id -> output block: contiguous ranges per XCD, grouped along N, M fastest
    const int total = NB * MB, L = blockIdx.x;
    const int P = total / 8;
    const int id = (L < 8 * P) ? (L % 8) * P + L / 8 : L;
    const int gsz = kGroupN * MB;
    const int grp = id / gsz, inb = id % gsz;
    const int nb0 = grp * kGroupN;
    const int gn = (NB - nb0 < kGroupN) ? (NB - nb0) : kGroupN;
    const int nb = nb0 + inb % gn, mb = inb / gn;

    Ctx<BK, HYB, BN, BM> C;
    C.values = a.values;
    C.meta = a.meta;
    C.ldw = a.ldw;
    C.N = a.N;
    C.n0 = (int64_t)nb * BN;
    C.W = HYB ? nullptr : a.W + C.n0 * a.ldw;
    C.r0 = 0;
    C.wave = wave;
    C.Tk = (int)(a.K / BK);
    const int64_t m0 = (int64_t)mb * BM;
    for (int v = 0; v < 2; ++v) {
        C.d_row[v] = 8 * (wave + 4 * v) + (lane >> 3);
        C.d_col[v] = (lane & 7) ^ ((C.d_row[v] >> 1) & 7);
    }
    C.s_row = 16 * wave + (lane >> 2);
    C.s_col = (lane & 3) ^ ((C.s_row >> 2) & 3);
    C.m_row = (64 * (wave & 1) + lane) >> 1;
    C.m_w = lane & 1;

    // ordered tile list of the tile row (dense first), tile columns kept for the X copies
    uint2* list = reinterpret_cast<uint2*>(smem + Lo::LIST);
    uint16_t* lcol = reinterpret_cast<uint16_t*>(smem + Lo::LCOL);
    int* wcount = reinterpret_cast<int*>(smem + Lo::WCNT);
    C.list = list;
    if (HYB) {
        const int tn = (int)(C.n0 / a.bn);
        const int rot = ROT ? tn : 0;
        const int t = tid;                         // one tile column per thread (Tk <= 256)
        hts_tile e = {0u, 0u, 0u, 0u};
        const bool have = t < C.Tk;
        if (have) e = a.index[(int64_t)tn * C.Tk + t];
        const bool isd = have && e.type == HTS_TILE_DENSE, iss = have && !isd;
        const uint64_t bd = __ballot(isd), bs = __ballot(iss);
        const int below_d = __builtin_amdgcn_mbcnt_hi((uint32_t)(bd >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bd, 0));
        const int below_s = __builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0));
        if (lane == 0) {
            wcount[wave] = __popcll(bd);
            wcount[4 + wave] = __popcll(bs);
        }
        __syncthreads();
        int nd = 0, pd = 0, ps = 0;
        for (int w = 0; w < 4; ++w) {
            nd += wcount[w];
            if (w < wave) {
                pd += wcount[w];
                ps += wcount[4 + w];
            }
        }
        if (have) {
            // each tile row starts its dense run and its 2:4 run at a different tile column, so
            // the tile rows running together spread their reads over the L2 channels
            const int ns = C.Tk - nd;
            const int pos = isd ? (pd + below_d + rot) % nd : nd + (ps + below_s + rot) % ns;
            list[pos] = uint2{e.val_off, e.meta_off};
            lcol[pos] = (uint16_t)t;
        }
        C.n_dense = nd;
        __syncthreads();
    } else {
        C.n_dense = C.Tk;
    }

    // per-lane X sources of this wave's copy jobs; the tile column is added per slice
    int64_t xrow[BM / 32];
    int xc[BM / 32];
#pragma unroll
    for (int v = 0; v < BM / 32; ++v) {
        const int row = 8 * (wave + 4 * v) + (lane >> 3);
        xc[v] = (lane & 7) ^ ((row >> 1) & 7);
        int64_t m = m0 + row;
        xrow[v] = (m < a.M ? m : a.M - 1) * a.ldx;   // rows past M only feed outputs that are not stored
    }
    auto set_x = [&](int ks) {
        const int p = ks / SPT, s = ks % SPT;
        const int tk = HYB ? (int)lcol[p] : p;
        const int64_t k0 = (int64_t)tk * BK + s * kKS;
#pragma unroll
        for (int v = 0; v < BM / 32; ++v) C.xsrc[v] = a.X + xrow[v] + k0 + 8 * xc[v];
    };

    f32x4 acc[4][NBJ];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) acc[b][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int S = C.Tk * SPT, Sd = C.n_dense * SPT;
    const bool wvalid = C.gvalid(wn);
    const int xoff = wm * WTM * 128;
    constexpr int PER_SLICE = BM / 32 + 2 * NG;     // copy instructions per wave per slice
    uint8_t* sink = smem + Lo::SINK;
    // prologue: slices 0 .. NSTAGE-2 in flight
#pragma unroll
    for (int k = 0; k < NSTAGE - 1; ++k) {
        if (k < S) {
            set_x(k);
            issue_slice<BK, HYB, BN, BM, NSTAGE>(C, k, smem + k * Lo::STAGE, sink);
        }
    }
    auto step = [&](int ks) {
        // wait until slice ks has landed: later slices (up to NSTAGE-2 of them) may stay in flight
        if (NSTAGE == 3 && ks + 1 < S) wait_vm<PER_SLICE>();
        else wait_vm<0>();
        __syncthreads();                    // everyone's copies landed; stage of slice ks-1 is free
        const int kn = ks + NSTAGE - 1;
        if (kn < S) {
            set_x(kn);
            issue_slice<BK, HYB, BN, BM, NSTAGE>(C, kn, smem + (kn % NSTAGE) * Lo::STAGE, sink);
        }
        return smem + (ks % NSTAGE) * Lo::STAGE;
    };
    int ks = 0;
    for (; ks < Sd; ++ks) {
        const uint8_t* st = step(ks);
        if (wvalid) compute_dense<T, SP, NBJ>(acc, st + xoff, st + Lo::WOFF + wn * kGroupBytes, lane);
    }
    for (; ks < S; ++ks) {
        const uint8_t* st = step(ks);
        if (wvalid)
            compute_sparse<T, SP, NBJ>(acc, st + xoff, st + Lo::WOFF + wn * kGroupBytes,
                                       reinterpret_cast<const uint32_t*>(st + Lo::MOFF + wn * kMetaGroupBytes), lane);
    }

    // epilogue: acc[b][bj] lane (j + 16q) holds Y^T rows 4q..4q+3 of block b, column j of block bj
    if (!wvalid) return;
    const int j = lane & 15, q = lane >> 4;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t n = C.n0 + 64 * wn + 16 * b + 4 * q;
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) {
            const int64_t m = m0 + wm * WTM + 16 * bj + j;
            if (m < a.M) store_y4(a.Y, m * a.ldy + n, a.y_dtype, acc[b][bj]);
        }
    }
}

template <typename T, int BK, bool HYB, int SP, int BN, int BM, int NSTAGE>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    using Lo = Layout<BN, BM, NSTAGE>;
    auto kern = gemm_prefill_kernel<T, BK, HYB, SP, BN, BM, NSTAGE>;
    static bool attr_set = false;   // per instantiation; raising the dynamic-LDS limit is idempotent
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Lo::TOTAL);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int NB = (int)((a.N + BN - 1) / BN), MB = (int)((a.M + BM - 1) / BM);
    kern<<<dim3((unsigned)(NB * MB)), dim3(kThreads), Lo::TOTAL, s>>>(a, NB, MB);
    return hipGetLastError();
}

template <typename T, int BK, bool HYB, int SP>
hipError_t launch4(const GemmArgs& a, int tile, hipStream_t s) {
    // one tile row per workgroup: BN = bn (a row-major weight uses 128-row blocks)
    // tile: 0 = 256 X rows, 3 stages; 1 = 128 rows, 2 stages; 2 = 128 rows, 3 stages
    const int bn = HYB ? a.bn : 128;
    if (bn == 64) {
        if (tile == 0) return launch_tile<T, BK, HYB, SP, 64, 256, 3>(a, s);
        if (tile == 1) return launch_tile<T, BK, HYB, SP, 64, 128, 2>(a, s);
        return launch_tile<T, BK, HYB, SP, 64, 128, 3>(a, s);
    }
    if (tile == 0) return launch_tile<T, BK, HYB, SP, 128, 256, 3>(a, s);
    if (tile == 1) return launch_tile<T, BK, HYB, SP, 128, 128, 2>(a, s);
    return launch_tile<T, BK, HYB, SP, 128, 128, 3>(a, s);
}

template <typename T, int BK, bool HYB>
hipError_t launch3(const GemmArgs& a, int sp, int tile, hipStream_t s) {
    return sp == SPARSE_SMFMAC ? launch4<T, BK, HYB, SPARSE_SMFMAC>(a, tile, s)
                               : launch4<T, BK, HYB, SPARSE_DECOMPRESS>(a, tile, s);
}

template <typename T>
hipError_t launch2(const GemmArgs& a, int sp, int tile, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128)
        return hyb ? launch3<T, 128, true>(a, sp, tile, s) : launch3<T, 128, false>(a, sp, tile, s);
    return hyb ? launch3<T, 64, true>(a, sp, tile, s) : launch3<T, 64, false>(a, sp, tile, s);
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, int sparse_path, int tile, hipStream_t s) {
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, sparse_path, tile, s)
                               : launch2<F16T>(a, sparse_path, tile, s);
}

}  // namespace hts
