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
// N-blocks (N fastest inside a group): blocks running together on one XCD share
// their W and X slices in its L2.
#include "gemm_common.h"

namespace hts {
namespace {

typedef __attribute__((address_space(3))) void lds_t;

constexpr int kKS = 64;                 // K elements per slice (16-bit elements: 128 bytes per row)
constexpr int kGroupBytes = 64 * 128;   // one 64-row weight group, dense (2:4 uses half)
constexpr int kMetaGroupBytes = 64 * 8; // codes of one 64-row group for one slice (16-bit elements)
// The single-tile-row kernel also takes 8-bit elements: a slice is always 128 bytes of every
// row (64 16-bit or 128 8-bit elements), so the LDS image of X and of the weights is the same;
// only the codes grow, to 16 bytes per row and slice.
template <int ES> constexpr int slice_k() { return 128 / ES; }
template <int ES> constexpr int meta_group_bytes() { return 64 * slice_k<ES>() / 8; }
constexpr int kMaxTileCols = 256;       // K/bk limit: the tile list of a tile row is kept in LDS
constexpr int kGroupN = 8;

// Block id -> output block (nb, mb).  ord = xcd | (gsn << 1) | (mfast << 6):
//   xcd   : 1 = each XCD (block id % 8) receives a contiguous range of the order below
//   gsn   : N-blocks per group (1..31); groups are walked in order
//   mfast : inside a group, 1 = M-blocks fastest, 0 = N-blocks fastest
// Default: contiguous per XCD, groups of 8 N-blocks, N fastest, so that the workgroups running
// together on one XCD cover about 8 N-blocks x 8 M-blocks and share W and X slices in its L2.
__device__ __forceinline__ void block_of(int L, int NB, int MB, int ord, int& nb, int& mb) {
    const int total = NB * MB;
    int id = L;
    if (ord & 1) {
        const int P = total / 8;
        id = (L < 8 * P) ? (L % 8) * P + L / 8 : L;
    }
    const int g = (ord >> 1) & 31, mfast = (ord >> 6) & 1;
    const int gsz = g * MB;
    const int grp = id / gsz, inb = id % gsz;
    const int nb0 = grp * g;
    const int gn = (NB - nb0 < g) ? (NB - nb0) : g;
    if (mfast) {
        nb = nb0 + inb / MB;
        mb = inb % MB;
    } else {
        nb = nb0 + inb % gn;
        mb = inb / gn;
    }
}

// LDS image of one stage: X slice (BM rows x 128 B), BN/64 weight groups, their codes.
template <int BN, int BM, int NSTAGE, int MGB = kMetaGroupBytes>
struct Layout {
    static constexpr int NG = BN / 64;
    static constexpr int WOFF = BM * 128;
    static constexpr int MOFF = WOFF + NG * kGroupBytes;
    static constexpr int STAGE = MOFF + NG * MGB;
    static constexpr int SINK = NSTAGE * STAGE;              // target of the padding copies
    static constexpr int LIST = SINK + 1024;                 // ordered tile list: {val_off, meta_off}
    static constexpr int LCOL = LIST + kMaxTileCols * 8;     // ... and the tile column of each entry
    static constexpr int WCNT = LCOL + kMaxTileCols * 2;     // dense tiles of each chunk (bytes)
    static constexpr int TOTAL = WCNT + 64;
};

// Dynamic LDS of the tiled kernels; copies address it by byte offset from an LDS-typed base,
// so no generic-to-LDS pointer conversion is needed per copy.
extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ lds_u8* lds_base() { return (lds_u8*)smem; }
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_off) {
    __builtin_amdgcn_global_load_lds(g, (lds_t*)(lds_base() + lds_off), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_off) {
    __builtin_amdgcn_global_load_lds(g, (lds_t*)(lds_base() + lds_off), 4, 0, 0);
}
// The same copies through a buffer resource: a scalar base and byte bound, a per-lane 32-bit
// offset fixed for the K loop and a scalar offset per slice -- no 64-bit address arithmetic per
// copy.  Lanes past the bound read zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ void buf16(rsrc_t r, uint32_t lds_off, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t*)(lds_base() + lds_off), 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void buf4(rsrc_t r, uint32_t lds_off, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_t*)(lds_base() + lds_off), 4, voff, soff, 0, 0);
}

// Everything the copy jobs need, fixed for the whole K loop.  A job moves 1 KiB (64
// lanes x 16 B) into contiguous LDS; each lane picks the global chunk whose swizzled
// LDS position is its slot.
template <int BK, bool HYB, int BN, int BM, int NW>
struct Ctx {
    static constexpr int NG = BN / 64;
    static constexpr int JPG = 8 / NW;  // copy jobs per 64-row group per wave
    static constexpr int XJ = BM / (8 * NW);  // X copy jobs per wave
    int64_t ldw;
    int64_t N, n0;
    int r0;                     // first row of the block inside its tile (0 when BN == bn)
    int wave, lane;
    uint32_t lnd;               // lane c: dense tiles of chunk c (they come first in the chunk)
    // the ordered list in registers, 64 entries per register (K / bk <= 256).  It is read in order,
    // and after each block of 64 entries the registers move down by one (shift_list), so entry p
    // is always lane p % 64 of the first register: one lane read, no register select.
    uint32_t lv[4], lm[4], lc[4];
    int Tk;
    rsrc_t xr;                          // X rows m0 .. M-1
    rsrc_t wr;                          // values of the tile row from its first tile (or W rows n0 ..)
    rsrc_t mr;                          // codes of the tile row from its first tile
    uint32_t vbase, mbase;              // first value / code word of the tile row
    uint32_t xso;                       // bytes: tile column and slice of the X copies of a slice
    uint32_t xvo[XJ];                   // per-lane byte offsets: X jobs
    uint32_t dvo[JPG];                  // dense group jobs (row * BK + chunk, or row * ldw + chunk)
    uint32_t svo;                       // 2:4 values job
    uint32_t mvo;                       // 2:4 codes job
    bool meta_to_sink;                  // a codes job past the codes of a slice repeats one into the sink
    int mjob;                           // this wave's codes job (256 bytes each)
    __device__ __forceinline__ bool gvalid(int gi) const { return n0 + 64 * gi < N; }
    __device__ __forceinline__ void shift_list() {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            lv[w] = lv[w + 1];
            lm[w] = lm[w + 1];
            lc[w] = lc[w + 1];
        }
        lv[3] = lm[3] = lc[3] = 0u;
    }
};

// Entry p of a list held one entry per lane (a uniform read: no LDS access); the caller has
// shifted the registers so that the block of entry p is in the first one.
__device__ __forceinline__ uint32_t list_entry(const uint32_t (&r)[4], int p) {
    return (uint32_t)__builtin_amdgcn_readlane((int)r[0], p & 63);
}

// Copies of one slice into an LDS stage.  Per 64-row weight group there are 8 copy jobs:
// dense = 8 x 1 KiB; 2:4 = 4 x 1 KiB of stored values, 2 x 256 B of codes and 2 padding copies
// of the codes into a sink.  Each of the NW waves issues BM/(8 NW) X copies and 8/NW copies per
// group for every slice, whatever the tile types, so the wait for one slice is a fixed count
// of outstanding copies.  KIND (dense / 2:4) is known at compile time: no branch per copy.
template <int BK, bool HYB, int BN, int BM, int NSTAGE, bool DENSE, int NW, int ES = 2>
__device__ __forceinline__ void issue_slice(const Ctx<BK, HYB, BN, BM, NW>& C, int ks, uint32_t stage) {
    constexpr int JPG = 8 / NW;
    constexpr int KSL = slice_k<ES>(), MGB = meta_group_bytes<ES>();
    using Lo = Layout<BN, BM, NSTAGE, MGB>;
    constexpr int SPT = BK / KSL;
    const int p = ks / SPT, s = ks % SPT;     // list position, slice of the tile
    // read the list entry before any copy is issued: an LDS read after a copy into LDS makes
    // the compiler wait for every copy in flight
    uint32_t voff = 0, moff = 0;
    if (HYB) {                                // every group of the block is in the same tile
        voff = list_entry(C.lv, p);
        moff = list_entry(C.lm, p);
    }
#pragma unroll
    for (int v = 0; v < BM / (8 * NW); ++v) buf16(C.xr, stage + 1024 * (C.wave + NW * v), C.xvo[v], C.xso);
#pragma unroll
    for (int gi = 0; gi < Lo::NG; ++gi) {
        const uint32_t ws = stage + Lo::WOFF + gi * kGroupBytes;
        if (!HYB) {                             // rows past N read zeros (bound of the resource)
#pragma unroll
            for (int v = 0; v < JPG; ++v)
                buf16(C.wr, ws + 1024 * (C.wave + NW * v), C.dvo[v],
                      (uint32_t)(ES * 64 * gi * C.ldw + 128 * (int64_t)ks));
            continue;
        }
        const uint32_t r = 64 * gi;             // a block is one tile row: groups at rows 0, 64
        if (DENSE) {
            // packed tile: slice s is chunk columns 8s .. 8s+7 of every row, 2048 bytes per 8 columns
            const uint32_t so = ES * (voff - C.vbase + r * BK) + 2048 * s;
#pragma unroll
            for (int v = 0; v < JPG; ++v) buf16(C.wr, ws + 1024 * (C.wave + NW * v), C.dvo[v], so);
        } else {
            // jobs 0-3: stored values; 4-7: codes, 256 bytes each (16-bit elements: two jobs of
            // codes, then the same two again into the sink).  With 4 waves wave w does jobs w and
            // 4 + w, with 8 waves job w.
            if (NW == 4 || C.wave < 4)
                buf16(C.wr, ws + 1024 * (C.wave & 3), C.svo, ES * (voff - C.vbase + r * (BK / 2)) + 1024 * s);
            if (NW == 4 || C.wave >= 4)
                buf4(C.mr,
                     C.meta_to_sink ? (uint32_t)Lo::SINK
                                    : stage + Lo::MOFF + gi * MGB + 256 * C.mjob,
                     C.mvo, 4 * (moff - C.mbase + r * (BK / 32) + (KSL / 32) * s));
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

// Weight fragments of row block b (16 rows) of a wave whose rows start at group g0: groups are
// 8 KiB apart in LDS, a dense group holds 64 rows x 128 B, a 2:4 group 64 rows x 64 B (+ codes).
// PANEL (packed weights): each 16-row block is the stored order of its slice -- chunk c of row i at
// (16 c + i) * 16, so a fragment read (16 rows of one chunk) is 256 contiguous bytes; otherwise
// (row-major W) row i at i * 128 with XOR-swizzled chunks, as for X.
template <typename T, int SP, int NBI, int NBJ, bool PANEL>
__device__ __forceinline__ void compute_dense(f32x4 (&acc)[NBI][NBJ], const uint8_t* xs, const uint8_t* ws, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int c0 = (SP == SPARSE_SMFMAC) ? g : 2 * g;
    const int c1 = (SP == SPARSE_SMFMAC) ? 4 + g : 2 * g + 1;
    const int a0 = PANEL ? 16 * (16 * c0 + i) : i * 128 + 16 * (c0 ^ ((i >> 1) & 7));
    const int a1 = PANEL ? 16 * (16 * c1 + i) : i * 128 + 16 * (c1 ^ ((i >> 1) & 7));
    u32x8 Bx[NBJ];
    load_x<SP, NBJ>(Bx, xs, lane);
    if constexpr (NBI == 4) {
        // every fragment of the slice is read before the first product: one LDS wait per slice
        u32x4 A[2][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int b = 0; b < 4; ++b) A[u][b] = ld16(ws + b * 2048 + (u ? a1 : a0));
        __builtin_amdgcn_sched_barrier(0);   // keep every read ahead of the products
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int bj = 0; bj < NBJ; ++bj)
                    acc[b][bj] = mfma_dense<T>(A[u][b], u ? hi4(Bx[bj]) : lo4(Bx[bj]), acc[b][bj]);
        return;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int h = 0; h < NBI / 4; ++h) {
            u32x4 A[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) A[b] = ld16(ws + (4 * h + b) * 2048 + (u ? a1 : a0));
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int bj = 0; bj < NBJ; ++bj)
                    acc[4 * h + b][bj] = mfma_dense<T>(A[b], u ? hi4(Bx[bj]) : lo4(Bx[bj]), acc[4 * h + b][bj]);
        }
    }
}

template <typename T, int SP, int NBI, int NBJ>
__device__ __forceinline__ void compute_sparse(f32x4 (&acc)[NBI][NBJ], const uint8_t* xs, const uint8_t* ws,
                                               const uint32_t* ms, int lane) {
    const int i = lane & 15, g = lane >> 4;
    const int s0 = 16 * (16 * g + i);    // stored order: chunk g of row i of the 16-row block
    u32x8 Bx[NBJ];
    load_x<SP, NBJ>(Bx, xs, lane);
#pragma unroll
    for (int h = 0; h < NBI / 4; ++h) {
        const uint8_t* wg = ws + h * kGroupBytes;
        const uint32_t* mg = ms + h * (meta_group_bytes<Elem<T>::bytes>() / 4);
        if (SP == SPARSE_SMFMAC) {
            u32x4 A[4];
            uint32_t idx[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                A[b] = ld16(wg + b * 1024 + s0);
                // 16-bit: a 16-bit half of the row's word g/2; 8-bit: the row's whole word g
                idx[b] = Elem<T>::bytes == 1 ? mg[4 * (16 * b + i) + g]
                                             : mg[2 * (16 * b + i) + (g >> 1)] >> (16 * (g & 1));
            }
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int bj = 0; bj < NBJ; ++bj)
                    acc[4 * h + b][bj] = mfma_sparse<T, 0>(A[b], Bx[bj], idx[b], acc[4 * h + b][bj]);
        } else {
            // expansion order: lane group g, substep u covers dense k [16g + 8u, +8) of the
            // slice = groups 4g + 2u, +1: stored bytes 16g + 8u of the row, codes at bit 16g + 8u
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                u32x4 A[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint2 v = *reinterpret_cast<const uint2*>(wg + b * 1024 + s0 + 8 * u);
                    const uint32_t code = (mg[2 * (16 * b + i) + (g >> 1)] >> (16 * (g & 1) + 8 * u)) & 0xFFu;
                    A[b] = expand_two_groups(v, code);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int bj = 0; bj < NBJ; ++bj)
                        acc[4 * h + b][bj] = mfma_dense<T>(A[b], u ? hi4(Bx[bj]) : lo4(Bx[bj]), acc[4 * h + b][bj]);
            }
        }
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt with vmcnt = N (low 4 bits and bits 14..15), expcnt and lgkmcnt left at their maxima
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until the oldest slice in flight has landed, leaving min(NSTAGE - 2, later) younger
// slices in flight (`later` = slices issued after it); each slice is PER copies per wave.
template <int NSTAGE, int PER>
__device__ __forceinline__ void wait_slice(int later) {
    const int k = later < NSTAGE - 2 ? later : NSTAGE - 2;
    if (NSTAGE >= 4 && k >= 2) wait_vm<(NSTAGE >= 4 ? 2 * PER : 0)>();
    else if (NSTAGE >= 3 && k >= 1) wait_vm<(NSTAGE >= 3 ? PER : 0)>();
    else wait_vm<0>();
}

template <typename T, int BK, bool HYB, int SP, int BN, int BM, int NSTAGE, int NW>
__global__ __launch_bounds__(64 * NW) void gemm_prefill_kernel(const GemmArgs a, int NB, int MB, int ord, int lch) {
    constexpr int ES = Elem<T>::bytes, KSL = slice_k<ES>(), MGB = meta_group_bytes<ES>();
    using Lo = Layout<BN, BM, NSTAGE, MGB>;
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    constexpr int NG = BN / 64, WM = NW / NG, WTM = BM / WM, NBJ = WTM / 16, SPT = BK / KSL;
    static_assert(NBJ >= 1 && BM % (8 * NW) == 0 && 2 * NW <= 16, "block shape");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave % NG, wm = wave / NG;

    // block id -> output block; blockIdx.y = part of the tile row's slices (split products)
    int nb, mb;
    block_of(blockIdx.x, NB, MB, ord, nb, mb);
    const int nsplit = a.nsplit > 1 ? a.nsplit : 1, split = (int)blockIdx.y;

    Ctx<BK, HYB, BN, BM, NW> C;
    C.ldw = a.ldw;
    C.N = a.N;
    C.n0 = (int64_t)nb * BN;
    C.r0 = 0;
    C.wave = wave;
    C.lane = lane;
    C.Tk = (int)(a.K / BK);
    const int64_t m0 = (int64_t)mb * BM;
    // copy sources: X rows m0 .. M-1 (rows past M read zeros and feed only unstored outputs);
    // the packed tile row from its first tile (offsets within a tile row fit 32 bits: K/bk <= 256
    // tiles of at most 32 KiB), or W rows n0 .. N-1 of the dense product
    // (byte addresses: the element pointers of GemmArgs are 16-bit typed, elements are ES bytes)
    const uint8_t* Xb = reinterpret_cast<const uint8_t*>(a.X);
    const uint8_t* Vb = reinterpret_cast<const uint8_t*>(a.values);
    const uint8_t* Wb = reinterpret_cast<const uint8_t*>(a.W);
    C.xr = make_rsrc(Xb + ES * m0 * a.ldx, (uint64_t)(a.M - m0) * a.ldx * ES);
    if (HYB) {
        const hts_tile first = a.index[(C.n0 / a.bn) * C.Tk];
        C.vbase = first.val_off;
        C.mbase = first.meta_off;
        C.wr = make_rsrc(Vb + (uint64_t)ES * C.vbase, (uint64_t)C.Tk * BN * BK * ES);
        C.mr = make_rsrc(a.meta + C.mbase, (uint64_t)C.Tk * BN * BK / 8);
    } else {
        C.vbase = C.mbase = 0;
        C.wr = make_rsrc(Wb + ES * C.n0 * a.ldw, (uint64_t)(a.N - C.n0) * a.ldw * ES);
        C.mr = C.wr;
    }
    C.xso = 0;
    for (int v = 0; v < 8 / NW; ++v) {
        const int row = 8 * (wave + NW * v) + (lane >> 3), col = (lane & 7) ^ ((row >> 1) & 7);
        // packed tile: a slice of a 16-row panel is one contiguous 2 KiB (its 8 chunk columns, the 16
        // rows consecutive in each), so job j copies kilobyte j % 2 of panel j / 2 straight -- the LDS
        // image is the stored order.  A row-major W: lane = (row, swizzled chunk) as for X.
        const int job = wave + NW * v;
        C.dvo[v] = HYB ? (uint32_t)((job >> 1) * 16 * BK * ES + 1024 * (job & 1) + 16 * lane)
                       : (uint32_t)(ES * (int64_t)row * a.ldw + 16 * col);
    }
    {
        // stored rows of BK/2 values: a slice of a 16-row panel is one contiguous kilobyte (job = panel)
        C.svo = (uint32_t)((wave & 3) * 16 * (BK / 2) * ES + 16 * lane);
        // codes jobs of 256 bytes: 64 rows x (KSL / 32) words per slice; job j covers words
        // 64 j .. 64 j + 63 of that row-major block
        constexpr int WPR = KSL / 32, NCJ = MGB / 256;
        const int cj = ((NW == 4) ? wave : wave - 4) & 3;  // this wave's codes job 0..3
        C.mjob = cj % NCJ;
        const int wi = 64 * C.mjob + lane;
        C.mvo = (uint32_t)(4 * ((wi / WPR) * (BK / 32) + (wi % WPR)));
        C.meta_to_sink = cj >= NCJ;
    }
    // ordered tile list of the tile row, tile columns kept for the X copies.  The row is cut
    // into chunks of 2^lch tile columns (inside one wave: lch <= 6), each ordered dense first.
    // Tile rows then walk K chunk by chunk, so workgroups of different tile rows that run
    // together stay within a chunk of each other and find each other's X slices in L2.
    uint2* list = reinterpret_cast<uint2*>(smem + Lo::LIST);
    uint16_t* lcol = reinterpret_cast<uint16_t*>(smem + Lo::LCOL);
    uint8_t* cnd = reinterpret_cast<uint8_t*>(smem + Lo::WCNT);   // dense tiles per chunk (<= 64 chunks)
    if (HYB) {
        const int tn = (int)(C.n0 / a.bn);
        const int t = tid;                         // one tile column per thread (Tk <= 256)
        hts_tile e = {0u, 0u, 0u, 0u};
        const bool have = t < C.Tk;
        if (have) e = a.index[(int64_t)tn * C.Tk + t];
        const bool isd = have && e.type == HTS_TILE_DENSE, iss = have && !isd;
        const uint64_t bd = __ballot(isd), bs = __ballot(iss);
        const int ch = 1 << lch, cl = lane & ~(ch - 1);             // first lane of this chunk
        const uint64_t cm = (lch == 6 ? ~0ull : ((1ull << ch) - 1)) << cl;
        const uint64_t lt = (1ull << lane) - 1;                      // lanes below this one
        const int nd_c = __popcll(bd & cm);
        const int below_d = __popcll(bd & cm & lt), below_s = __popcll(bs & cm & lt);
        if (have) {
            const int pos = (t & ~(ch - 1)) + (isd ? below_d : nd_c + below_s);
            list[pos] = uint2{e.val_off, e.meta_off};
            lcol[pos] = (uint16_t)t;
            if (lane == cl) cnd[t >> lch] = (uint8_t)nd_c;
        }
        __syncthreads();
        const int nch = (C.Tk + ch - 1) >> lch;
        C.lnd = lane < nch ? (uint32_t)cnd[lane] : 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int q = 64 * w + lane;
            const bool in = q < C.Tk;
            C.lv[w] = in ? list[q].x : 0u;
            C.lm[w] = in ? list[q].y : 0u;
            C.lc[w] = in ? (uint32_t)lcol[q] : 0u;
        }
    } else {
        C.lnd = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) C.lv[w] = C.lm[w] = C.lc[w] = 0u;
    }

    // per-lane X sources of this wave's copy jobs; the tile column is added per slice
    constexpr int XJ = BM / (8 * NW);      // X copy jobs per wave
#pragma unroll
    for (int v = 0; v < XJ; ++v) {
        const int row = 8 * (wave + NW * v) + (lane >> 3);
        const int xc = (lane & 7) ^ ((row >> 1) & 7);
        C.xvo[v] = (uint32_t)(ES * (int64_t)row * a.ldx + 16 * xc);
    }
    auto set_x = [&](int ks) {
        const int p = ks / SPT, s = ks % SPT;
        const int tk = HYB ? (int)list_entry(C.lc, p) : p;
        C.xso = (uint32_t)(ES * tk * BK + 128 * s);
    };

    f32x4 acc[4][NBJ];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) acc[b][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

    // slices k0 .. k1-1 of the ordered list (all of them unless the product is split)
    const int S = C.Tk * SPT, lcs = lch + (SPT == 2 ? 1 : 0);   // slices per chunk: 2^lcs
    // slice kn is dense when it lies in the dense run at the start of its chunk
    auto dense_slice = [&](int kn) {
        return !HYB || (kn & ((1 << lcs) - 1)) < SPT * (int)__builtin_amdgcn_readlane((int)C.lnd, kn >> lcs);
    };
    const int k0 = (int)((int64_t)split * S / nsplit), k1 = (int)((int64_t)(split + 1) * S / nsplit);
    const bool wvalid = C.gvalid(wn);
    const int xoff = wm * WTM * 128;
    constexpr int PER_SLICE = XJ + NG * (8 / NW);   // copy instructions per wave per slice
    if (HYB)                                         // bring the block of list entry k0 / SPT first
        for (int b = 0; b < k0 / (64 * SPT); ++b) C.shift_list();
    auto issue = [&](int kn) {   // called for kn = k0, k0 + 1, ... in order
        if (HYB && kn > k0 && kn % (64 * SPT) == 0) C.shift_list();
        set_x(kn);
        const uint32_t stage = (kn % NSTAGE) * Lo::STAGE;
        if (dense_slice(kn)) issue_slice<BK, HYB, BN, BM, NSTAGE, true, NW, ES>(C, kn, stage);
        else issue_slice<BK, HYB, BN, BM, NSTAGE, false, NW, ES>(C, kn, stage);
    };
    // prologue: slices k0 .. k0+NSTAGE-2 in flight
#pragma unroll
    for (int k = 0; k < NSTAGE - 1; ++k)
        if (k0 + k < k1) issue(k0 + k);
    auto step = [&](int ks) {
        // wait until slice ks has landed: later slices (up to NSTAGE-2 of them) may stay in flight
        wait_slice<NSTAGE, PER_SLICE>(k1 - 1 - ks);
        __syncthreads();                    // everyone's copies landed; stage of slice ks-1 is free
        const int kn = ks + NSTAGE - 1;
        if (kn < k1) issue(kn);
        return smem + (ks % NSTAGE) * Lo::STAGE;
    };
    int ks = k0;
    if constexpr (!HYB) {
        for (; ks < k1; ++ks) {
            const uint8_t* st = step(ks);
            if (wvalid) compute_dense<T, SP, 4, NBJ, false>(acc, st + xoff, st + Lo::WOFF + wn * kGroupBytes, lane);
        }
    } else {
        // chunk by chunk: its dense run, then its 2:4 run (a split part may start or end inside)
        while (ks < k1) {
            const int c = ks >> lcs, cs = c << lcs;
            const int ce = (cs + (1 << lcs)) < k1 ? cs + (1 << lcs) : k1;
            int de = cs + SPT * (int)__builtin_amdgcn_readlane((int)C.lnd, c);
            de = de < ce ? de : ce;
            for (; ks < de; ++ks) {
                const uint8_t* st = step(ks);
                if (wvalid) compute_dense<T, SP, 4, NBJ, true>(acc, st + xoff, st + Lo::WOFF + wn * kGroupBytes, lane);
            }
            for (; ks < ce; ++ks) {
                const uint8_t* st = step(ks);
                if (wvalid)
                    compute_sparse<T, SP, 4, NBJ>(acc, st + xoff, st + Lo::WOFF + wn * kGroupBytes,
                                               reinterpret_cast<const uint32_t*>(st + Lo::MOFF + wn * MGB), lane);
            }
        }
    }

    // epilogue: acc[b][bj] lane (j + 16q) holds Y^T rows 4q..4q+3 of block b, column j of block bj;
    // a split product writes its fp32 part instead (rows of N floats)
    if (!wvalid) return;
    void* out = a.Y;
    int64_t ldo = a.ldy;
    int32_t odt = a.y_dtype;
    if (nsplit > 1) {
        out = a.part + (int64_t)split * a.M * a.N;
        ldo = a.N;
        odt = HTS_F32;
    }
    const int j = lane & 15, q = lane >> 4;
    if (a.gate && nsplit == 1) {
        // gated output (a split product applies the gate in the sum of its parts): every gate value
        // of the lane is loaded before the first store, since G may be Y
        f32x4 gv[4][NBJ];
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int bj = 0; bj < NBJ; ++bj) {
                const int64_t m = m0 + wm * WTM + 16 * bj + j, n = C.n0 + 64 * wn + 16 * b + 4 * q;
                gv[b][bj] = m < a.M ? load_gate4(a.gate, m * a.ldg + n, a.y_dtype) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int bj = 0; bj < NBJ; ++bj) acc[b][bj] = silu_times4(gv[b][bj], acc[b][bj]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int64_t n = C.n0 + 64 * wn + 16 * b + 4 * q;
#pragma unroll
        for (int bj = 0; bj < NBJ; ++bj) {
            const int64_t m = m0 + wm * WTM + 16 * bj + j;
            if (m < a.M) store_y4(out, m * ldo + n, odt, acc[b][bj]);
        }
    }
}

// Sum of the parts of a split product, in part order (deterministic), rounded once to y_dtype.
// One thread per 4 consecutive outputs of a row (N is a multiple of 64).
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, int nsplit, const void* gate,
                                                        int64_t ldg, int64_t M,
                                                        int64_t N, void* Y, int64_t ldy, int32_t y_dtype) {
    const int64_t nq = N / 4;
    const int64_t qi = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (qi >= M * nq) return;
    const int64_t m = qi / nq, n = 4 * (qi % nq);
    f32x4 acc = *reinterpret_cast<const f32x4*>(part + m * N + n);
    for (int i = 1; i < nsplit; ++i) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(part + ((int64_t)i * M + m) * N + n);
        acc = f32x4{acc[0] + v[0], acc[1] + v[1], acc[2] + v[2], acc[3] + v[3]};
    }
    if (gate) acc = silu_times4(load_gate4(gate, m * ldg + n, y_dtype), acc);
    store_y4(Y, m * ldy + n, y_dtype, acc);
}

// Block order of the tiled kernels (HTS_PREFILL_ORDER overrides; see block_of).
int prefill_order() {
    const char* e = getenv("HTS_PREFILL_ORDER");
    const int v = (e && *e) ? atoi(e) : -1;
    const int g = (v >> 1) & 31;
    if (v < 0 || v > 127 || g == 0) return 1 | (kGroupN << 1);   // groups of at least one N-block
    return v;
}

// Tile columns per chunk of the ordered list, as log2: chunks of 512 K by default
// (HTS_PREFILL_CHUNK = 4, 8, 16, 32 or 64 tile columns overrides).
int prefill_chunk_log2(int bk) {
    const char* e = getenv("HTS_PREFILL_CHUNK");
    const int v = (e && *e) ? atoi(e) : 512 / bk;
    for (int l = 2; l <= 6; ++l)
        if (v == (1 << l)) return l;
    return bk == 64 ? 3 : 2;
}

template <typename T, int BK, bool HYB, int SP, int BN, int BM, int NSTAGE, int NW = 4>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    using Lo = Layout<BN, BM, NSTAGE, meta_group_bytes<Elem<T>::bytes>()>;
    auto kern = gemm_prefill_kernel<T, BK, HYB, SP, BN, BM, NSTAGE, NW>;
    static bool attr_set = false;   // per instantiation; raising the dynamic-LDS limit is idempotent
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Lo::TOTAL);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int NB = (int)((a.N + BN - 1) / BN), MB = (int)((a.M + BM - 1) / BM);
    const int nsplit = a.nsplit > 1 ? a.nsplit : 1;
    kern<<<dim3((unsigned)(NB * MB), (unsigned)nsplit), dim3(64 * NW), Lo::TOTAL, s>>>(a, NB, MB, prefill_order(),
                                                                                   prefill_chunk_log2(BK));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    const int64_t quads = a.M * (a.N / 4);
    split_sum_kernel<<<dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s>>>(a.part, nsplit, a.gate, a.ldg, a.M, a.N, a.Y,
                                                                              a.ldy, a.y_dtype);
    return hipGetLastError();
}

template <typename T, int BK, bool HYB, int SP>
hipError_t launch4(const GemmArgs& a, hipStream_t s) {
    // one tile row x 128 X rows per workgroup, 4 waves, 2 stages (two workgroups per CU)
    if constexpr (Elem<T>::bytes == 1) {
        return launch_tile<T, BK, HYB, SP, 128, 128, 2>(a, s);
    } else {
        if (HYB && a.bn == 64) return launch_tile<T, BK, HYB, SP, 64, 128, 2>(a, s);
        return launch_tile<T, BK, HYB, SP, 128, 128, 2>(a, s);
    }
}

template <typename T, int BK, bool HYB>
hipError_t launch3(const GemmArgs& a, int sp, hipStream_t s) {
    if constexpr (Elem<T>::bytes == 1) {
        (void)sp;
        return launch4<T, BK, HYB, SPARSE_SMFMAC>(a, s);   // 8-bit: no expansion path
    } else {
        return sp == SPARSE_SMFMAC ? launch4<T, BK, HYB, SPARSE_SMFMAC>(a, s)
                                   : launch4<T, BK, HYB, SPARSE_DECOMPRESS>(a, s);
    }
}

template <typename T>
hipError_t launch2(const GemmArgs& a, int sp, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128) return hyb ? launch3<T, 128, true>(a, sp, s) : launch3<T, 128, false>(a, sp, s);
    return hyb ? launch3<T, 64, true>(a, sp, s) : launch3<T, 64, false>(a, sp, s);
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, int sparse_path, hipStream_t s) {
    if (a.dtype == HTS_FP8_E4M3)   // 128x128 tiles only
        return a.index ? launch3<FP8T, 128, true>(a, sparse_path, s) : launch3<FP8T, 128, false>(a, sparse_path, s);
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, sparse_path, s) : launch2<F16T>(a, sparse_path, s);
}

}  // namespace hts
