// Pieces shared by the tiled (large-M) product kernels: LDS layout of a stage, the copies of a
// weight slice (and of an X slice) from global memory into LDS, the ordered tile list of a tile
// row, the workgroup order, and explicit waits on outstanding copies.
#pragma once

#include "gemm_common.h"

namespace hts {
namespace {

typedef __attribute__((address_space(3))) void lds_t;

constexpr int kGroupBytes = 64 * 128;   // one 64-row weight group, dense (2:4 uses half)
constexpr int kMetaGroupBytes = 64 * 8; // codes of one 64-row group for one slice (16-bit elements)
// The single-tile-row kernel also takes 8-bit elements: a slice is always 128 bytes of every
// row (64 16-bit or 128 8-bit elements), so the LDS image of X and of the weights is the same;
// only the codes grow, to 16 bytes per row and slice.
template <int ES> constexpr int slice_k() { return 128 / ES; }
template <int ES> constexpr int meta_group_bytes() { return 64 * slice_k<ES>() / 8; }
constexpr int kMaxTileCols = 256;       // K/bk limit: the tile list of a tile row is kept in LDS
constexpr int kGroupN = 8;              // N-blocks per group of the block order (16-bit data)
constexpr int kGroupN8 = 11;            // ... and for 8-bit data

// Block id -> output block (nb, mb).  ord = xcd | (gsn << 1) | (mfast << 6):
//   xcd   : 1 = each XCD (block id % 8) receives a contiguous range of the order below
//   gsn   : N-blocks per group (1..31); groups are walked in order
//   mfast : inside a group, 1 = M-blocks fastest, 0 = N-blocks fastest
// Default: contiguous per XCD, groups of 8 N-blocks (11 for 8-bit data), N fastest, so that the
// workgroups running together on one XCD cover about 8 N-blocks x 8 M-blocks and share W and X
// slices in its L2.
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

// LDS image of one stage: X slice (BM rows x 128 B), then BN/64 weight-group slots of 8 KiB.  A
// dense group fills its slot; a 2:4 group's stored values fill the lower half and its codes (one
// 1 KiB job: 64 code rows) sit in the upper half, so the codes need no space of their own.  The ordered tile list
// is built once, before the first copy, in stage 0's memory.  With two stages nothing else is
// needed: a 128 x 192 block then takes 80 KiB, and two such workgroups fit in a CU's 160 KiB.
template <int BN, int BM, int NSTAGE, int MGB = kMetaGroupBytes>
struct Layout {
    static constexpr int NG = BN / 64;
    static constexpr int WOFF = BM * 128;
    static constexpr int MHALF = kGroupBytes / 2;            // codes inside a 2:4 group's slot
    static constexpr int STAGE = WOFF + NG * kGroupBytes;
    static constexpr int SINK = NSTAGE * STAGE;              // target of the padding copies (3+ stages)
    static constexpr int TOTAL = SINK + (NSTAGE > 2 ? 1024 : 0);
    static constexpr int LIST = 0;                           // ordered tile list: {val_off, meta_off}
    static constexpr int LCOL = LIST + kMaxTileCols * 8;     // ... and the tile column of each entry
    static constexpr int WCNT = LCOL + kMaxTileCols * 2;     // dense tiles of each chunk (bytes)
    static_assert(MGB <= 1024 && 1024 <= MHALF, "a group's codes job fits the upper half of a 2:4 group's slot");
    static_assert(WCNT + 64 <= STAGE, "the list fits in stage 0");
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

// Blocks of two 64-row tile rows (64-row tiles): Ctx's lv / lm then hold the first row's records in
// K order and lc both rows' types (bit 0: first row 2:4, bit 1: second); the second row's records
// are kept here, one tile column per lane, and move along with Ctx's (shift with shift_list).
struct SecondRow {
    uint32_t lv[4], lm[4];
    __device__ __forceinline__ void shift() {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            lv[w] = lv[w + 1];
            lm[w] = lm[w + 1];
        }
        lv[3] = lm[3] = 0u;
    }
};

// Entry p of a list held one entry per lane (a uniform read: no LDS access); the caller has
// shifted the registers so that the block of entry p is in the first one.
__device__ __forceinline__ uint32_t list_entry(const uint32_t (&r)[4], int p) {
    return (uint32_t)__builtin_amdgcn_readlane((int)r[0], p & 63);
}

// Copies of one slice into an LDS stage.  Per 64-row weight group: dense = 8 jobs of 1 KiB; 2:4 =
// 4 x 1 KiB of stored values and one 1 KiB job of codes.  With three or more stages the waves
// that copy no codes pad with a copy into a sink: each of the NW waves then issues BM/(8 NW) X
// copies and 8/NW copies per group for every slice, whatever the tile types, so the wait for one
// slice is a fixed count of outstanding copies.  Two stages wait for every copy in flight, so
// they skip the padding.  KIND (dense / 2:4) is known at compile time: no branch per copy.
// The codes of 2:4 group gi (rows r .. r+63 of the tile whose codes start at word moff) into the
// upper half of its LDS slot ws.  One job of 16 bytes per lane: lane L copies code row L of the
// group, all BK/32 words of it (the codes of every slice of the tile: a slice reads its own words
// of each row; with 2 words per row the job's second half holds the next rows, unused).  One
// wave per group issues it; with three or more stages the others pad with a copy into the sink,
// so every wave issues the same number of copies per slice.  Against copying only the slice's
// words in 4-byte-per-lane jobs (two per slice for 16-bit data, four for 8-bit), bit-identical
// results and 1.00-1.02x the speed (most on layers with many 2:4 tiles).
template <int BK, bool HYB, int BN, int BM, int NSTAGE, int NW, int ES>
__device__ __forceinline__ void issue_codes(const Ctx<BK, HYB, BN, BM, NW>& C, int gi, uint32_t r, uint32_t moff,
                                            int s, uint32_t ws) {
    using Lo = Layout<BN, BM, NSTAGE, meta_group_bytes<ES>()>;
    (void)s;
    if (C.wave == NW - Lo::NG + gi)
        buf16(C.mr, ws + Lo::MHALF, C.mvo, 4 * (moff - C.mbase + r * (BK / 32)));
    else if (NSTAGE > 2 && (NW == 4 || C.wave >= 4))
        buf4(C.mr, (uint32_t)Lo::SINK, 0u, 4 * (moff - C.mbase));
}

template <int BK, bool HYB, int BN, int BM, int NW>
__device__ __forceinline__ void issue_x(const Ctx<BK, HYB, BN, BM, NW>& C, uint32_t stage) {
#pragma unroll
    for (int v = 0; v < BM / (8 * NW); ++v) buf16(C.xr, stage + 1024 * (C.wave + NW * v), C.xvo[v], C.xso);
}

// Pieces of issue_slice (below) for blocks of two tile rows: the X copies of a slice, and group gi
// of a slice from a packed tile -- rows r .. r+63 of the tile whose values start at element voff
// and whose codes start at word moff; s = slice of the tile.  (issue_slice keeps its own copy of
// this code: written inline there, the single-tile-row kernels compile as before.)
template <int BK, bool HYB, int BN, int BM, int NSTAGE, bool DENSE, int NW, int ES>
__device__ __forceinline__ void issue_packed_group(const Ctx<BK, HYB, BN, BM, NW>& C, int gi, uint32_t r,
                                                   uint32_t voff, uint32_t moff, int s, uint32_t stage) {
    constexpr int JPG = 8 / NW;
    constexpr int KSL = slice_k<ES>(), MGB = meta_group_bytes<ES>();
    using Lo = Layout<BN, BM, NSTAGE, MGB>;
    const uint32_t ws = stage + Lo::WOFF + gi * kGroupBytes;
    if (DENSE) {
        // packed tile: slice s is chunk columns 8s .. 8s+7 of every row, 2048 bytes per 8 columns
        const uint32_t so = ES * (voff - C.vbase + r * BK) + 2048 * s;
#pragma unroll
        for (int v = 0; v < JPG; ++v) buf16(C.wr, ws + 1024 * (C.wave + NW * v), C.dvo[v], so);
    } else {
        // jobs 0-3: stored values (wave w's, or waves 0-3's with 8 waves); then the group's codes,
        // one job from one wave (issue_codes)
        if (NW == 4 || C.wave < 4)
            buf16(C.wr, ws + 1024 * (C.wave & 3), C.svo, ES * (voff - C.vbase + r * (BK / 2)) + 1024 * s);
        issue_codes<BK, HYB, BN, BM, NSTAGE, NW, ES>(C, gi, r, moff, s, ws);
    }
}

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
            // jobs 0-3: stored values (wave w's, or waves 0-3's with 8 waves); then the group's
            // codes, one job from one wave (issue_codes)
            if (NW == 4 || C.wave < 4)
                buf16(C.wr, ws + 1024 * (C.wave & 3), C.svo, ES * (voff - C.vbase + r * (BK / 2)) + 1024 * s);
            issue_codes<BK, HYB, BN, BM, NSTAGE, NW, ES>(C, gi, r, moff, s, ws);
        }
    }
}

// Copies of one slice of a block of two 64-row tile rows (16-bit data, two stages): the slice's
// tile column is the same in both rows, each row's tile has its own type and offsets, and a
// second row past N is not copied.
template <int BK, bool HYB, int BN, int BM, int NW>
__device__ __forceinline__ void issue_slice_two(const Ctx<BK, HYB, BN, BM, NW>& C, const SecondRow& R2, int ks,
                                                uint32_t stage) {
    static_assert(BN == 128, "two 64-row groups");
    constexpr int SPT = BK / 64;
    const int p = ks / SPT, s = ks % SPT;
    // every list read before the first copy
    const uint32_t ty = list_entry(C.lc, p);
    const uint32_t v0 = list_entry(C.lv, p), m0 = list_entry(C.lm, p);
    const uint32_t v1 = list_entry(R2.lv, p), m1 = list_entry(R2.lm, p);
    issue_x(C, stage);
    if (ty & 1u) issue_packed_group<BK, HYB, BN, BM, 2, false, NW, 2>(C, 0, 0u, v0, m0, s, stage);
    else issue_packed_group<BK, HYB, BN, BM, 2, true, NW, 2>(C, 0, 0u, v0, m0, s, stage);
    if (C.gvalid(1)) {
        if (ty & 2u) issue_packed_group<BK, HYB, BN, BM, 2, false, NW, 2>(C, 1, 0u, v1, m1, s, stage);
        else issue_packed_group<BK, HYB, BN, BM, 2, true, NW, 2>(C, 1, 0u, v1, m1, s, stage);
    }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt with vmcnt = N (low 4 bits and bits 14..15), expcnt and lgkmcnt left at their maxima
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Reads the tile row's index records (one tile column per thread: K / bk <= 256 <= threads) and
// leaves the ordered list in C's registers: the row cut into chunks of 2^lch tile columns (inside
// one wave: lch <= 6), each ordered dense first; C.lnd lane c = dense tiles of chunk c.  Tile rows
// then walk K chunk by chunk, so workgroups of different tile rows that run together stay within a
// chunk of each other and find each other's X slices in L2.  Uses LDS at Lo::LIST .. Lo::WCNT + 64
// (stage 0's memory): it ends with a barrier, so no copy into that stage starts before every
// wave has read the list.
template <typename Lo, int BK, bool HYB, int BN, int BM, int NW>
__device__ __forceinline__ void load_tile_list(Ctx<BK, HYB, BN, BM, NW>& C, const GemmArgs& a, int lch, int tid,
                                               int lane) {
    uint2* list = reinterpret_cast<uint2*>(smem + Lo::LIST);
    uint16_t* lcol = reinterpret_cast<uint16_t*>(smem + Lo::LCOL);
    uint8_t* cnd = reinterpret_cast<uint8_t*>(smem + Lo::WCNT);   // dense tiles per chunk (<= 64 chunks)
    const int tn = (int)(C.n0 / a.bn);
    const int t = tid;
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
    __syncthreads();   // the list area is stage 0: every wave has read it before the first copy
}

// Reads the index records of the block's two 64-row tile rows (one tile column per thread) and
// leaves them in registers in K order: C.lv / C.lm the first row's {val_off, meta_off}, R2 the
// second's (zeros when that row is past N), C.lc the two types.  Uses stage 0's memory and ends
// with a barrier, as load_tile_list.
template <typename Lo, int BK, bool HYB, int BN, int BM, int NW>
__device__ __forceinline__ void load_two_lists(Ctx<BK, HYB, BN, BM, NW>& C, SecondRow& R2, const GemmArgs& a, int tid,
                                               int lane) {
    uint2* l0 = reinterpret_cast<uint2*>(smem + Lo::LIST);
    uint2* l1 = reinterpret_cast<uint2*>(smem + Lo::LIST + kMaxTileCols * 8);
    uint8_t* ty = reinterpret_cast<uint8_t*>(smem + Lo::LIST + 2 * kMaxTileCols * 8);
    static_assert(Lo::LIST + 2 * kMaxTileCols * 8 + kMaxTileCols <= Lo::STAGE, "both lists fit in stage 0");
    const int64_t tn = C.n0 / a.bn;                  // the first of the two tile rows
    const bool second = C.gvalid(1);
    if (tid < C.Tk) {
        const hts_tile e0 = a.index[tn * C.Tk + tid];
        hts_tile e1 = {0u, 0u, 0u, 0u};
        if (second) e1 = a.index[(tn + 1) * C.Tk + tid];
        l0[tid] = uint2{e0.val_off, e0.meta_off};
        l1[tid] = uint2{e1.val_off, e1.meta_off};
        ty[tid] = (uint8_t)((e0.type != HTS_TILE_DENSE ? 1u : 0u) | (second && e1.type != HTS_TILE_DENSE ? 2u : 0u));
    }
    __syncthreads();
    C.lnd = 0u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int q = 64 * w + lane;
        const bool in = q < C.Tk;
        C.lv[w] = in ? l0[q].x : 0u;
        C.lm[w] = in ? l0[q].y : 0u;
        R2.lv[w] = in ? l1[q].x : 0u;
        R2.lm[w] = in ? l1[q].y : 0u;
        C.lc[w] = in ? (uint32_t)ty[q] : 0u;
    }
    __syncthreads();   // stage 0: every wave has read the lists before the first copy
}

}  // namespace

// Host side (gemm_prefill.hip): tile columns per dense-first chunk of the ordered list, as log2.
int prefill_chunk_log2(int bk);

}  // namespace hts
