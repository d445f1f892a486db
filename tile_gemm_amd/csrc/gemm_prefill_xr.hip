// Hybrid tile-sparse product for large M with X in registers: the matrix-core-bound tiled path of
// unsplit products on 128-row tiles (and of the same-library dense product).
//
// A workgroup of 4 waves owns one tile row (128 weight rows) x 256 X rows of Y^T and walks K in
// 64-wide slices (128 bytes of every row).  Wave w owns X rows 64w .. 64w+63 of the block, which no
// other wave reads, so its X fragments go from global memory straight into registers in the
// matrix-core operand layout, one slice ahead; only the weight slice -- shared by the four waves --
// is copied into LDS (global-to-LDS copies, three stages).  Per slice a wave reads the 16 weight
// fragments of its 8 row blocks from LDS and feeds 8 x 4 blocks of 16 x 16 outputs (accumulators in
// the matrix-core register file), so the LDS carries only the weight and the copy path moves a
// third less per flop than with both operands staged.  Dense tiles go to the 16x16x32 MFMA, 2:4
// tiles to the 16x16x64 SMFMAC (or in-register expansion to dense MFMA), into one accumulator per
// output block (page "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", section 2, inference
// and deployment; execution tiles of 128 x 128 and larger, sections 2 and 4).  The tile row's list
// is walked in dense-first chunks as in the LDS-staged kernel.
//
// Slice schedule of a wave (step ks): wait for its own copies of slice ks and its X loads of slice
// ks; LDS-only workgroup barrier; read all weight fragments of slice ks from LDS; issue the X loads
// of slice ks+1 and the copies of slice ks+2 while those reads are in flight; then the products.
#include <cstring>
#include <type_traits>

#include "prefill_common.h"

namespace hts {
namespace {

// Workgroup barrier that orders LDS only.  __syncthreads() is a workgroup-scope fence on every
// address space, which on this chip waits for all of the wave's vector memory operations -- the X
// loads and weight copies of later slices included -- and so would drain the pipeline at every
// slice.  Here each wave waits for its own copies of the slice explicitly (vmcnt), then this
// barrier: its own LDS reads of the stage about to be overwritten complete first (release), and no
// LDS read moves above it (acquire).
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// X fragments of one slice for a wave's four 16-row blocks, from X rearranged into 16-row panels
// (chunk c of panel row j at (16 c + j) * 16 bytes from the panel start): lane j + 16 g takes chunks
// c0(g) and c1(g) of row j of the slice.  In the sparse-instruction order (c0 = g, c1 = 4 + g) each
// load is one contiguous kilobyte.  Panels past the packed rows read zeros (resource bound).
template <int SP>
__device__ __forceinline__ void load_xr(u32x8 (&B)[4], rsrc_t xr, const uint32_t (&xv)[4], uint32_t so) {
    constexpr uint32_t dch = SP == SPARSE_SMFMAC ? 1024u : 256u;   // (c1 - c0) * 256 bytes
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) {
        const u32x4 lo = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xv[bj], so, 0));
        const u32x4 hi = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xv[bj] + dch, so, 0));
        B[bj] = cat8(lo, hi);
    }
}

// Half-slice software pipeline.  A slice is fed to the matrix cores in two halves -- dense: the
// two 32-deep substeps over all 8 row blocks (32 MFMA each); 2:4: row blocks 0-3, then 4-7 (16
// SMFMAC each) -- and the weight fragments of each half are read from LDS during the previous
// half, so no product waits for LDS.  Fragment registers have one shape for both tile types (8
// value kilobytes and 4 code words; a 2:4 half uses 4 + 4, and its other reads repeat those), so a
// half of either type can follow a half of the other with no register copies.
struct Frags {
    u32x4 a[8];
    uint32_t idx[4];
};

// Reads the fragments of half h of the slice in the LDS stage `ws` (codes at ws + 2 groups).
// PANEL: packed stored order (chunk c of row i at (16 c + i) * 16); otherwise row-major W with
// XOR-swizzled chunks (dense only).
template <typename T, int SP, bool PANEL, int h>
__device__ __forceinline__ void read_half(Frags& F, const uint8_t* ws, bool dense, int lane) {
    constexpr int MW = meta_group_bytes<Elem<T>::bytes>() / 4;   // code words of a 64-row group
    const int i = lane & 15, g = lane >> 4;
    const int c = (SP == SPARSE_SMFMAC) ? (h ? 4 + g : g) : (2 * g + h);
    const int ad = PANEL ? 16 * (16 * c + i) : i * 128 + 16 * (c ^ ((i >> 1) & 7));
    const int as = h * kGroupBytes + 16 * (16 * g + i);        // 2:4 values: chunk g of row i of block b
    const uint32_t* ms = reinterpret_cast<const uint32_t*>(ws + 2 * kGroupBytes) + h * MW;
#pragma unroll
    for (int b = 0; b < 8; ++b) F.a[b] = ld16(ws + (dense ? b * 2048 + ad : (b & 3) * 1024 + as));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int r = 16 * b + i;
        // 16-bit: a 16-bit half of the row's word g/2 (SMFMAC) or the row's word g/2 (expansion,
        // both halves); 8-bit: the row's whole word g
        F.idx[b] = Elem<T>::bytes == 1 ? ms[4 * r + g] : ms[2 * r + (g >> 1)];
    }
}

// Products of half h (dense: substep u = h) with X fragments B.
// Products of half h (dense: substep u = h) with X fragments B, for fragment rows [R0, R1) of the
// half (dense: row blocks R0..R1-1 of 8; 2:4: row blocks 4h + R0 .. of 4, R1 <= 4).
template <typename T, int SP, bool DENSE, int h, int R0, int R1>
__device__ __forceinline__ void mma_part(f32x4 (&acc)[8][4], const Frags& F, const u32x8 (&B)[4], int lane) {
    const int g = lane >> 4;
    if constexpr (DENSE) {
#pragma unroll
        for (int b = R0; b < R1; ++b)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                acc[b][bj] = mfma_dense<T>(F.a[b], h ? hi4(B[bj]) : lo4(B[bj]), acc[b][bj]);
    } else if constexpr (SP == SPARSE_SMFMAC) {
#pragma unroll
        for (int b = R0; b < R1; ++b) {
            const uint32_t idx = Elem<T>::bytes == 1 ? F.idx[b] : F.idx[b] >> (16 * (g & 1));
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                acc[4 * h + b][bj] = mfma_sparse<T, 0>(F.a[b], B[bj], idx, acc[4 * h + b][bj]);
        }
    } else {
        // expansion order: lane group g, substep u covers dense k [16g + 8u, +8) of the slice =
        // groups 4g + 2u, +1: stored bytes 16g + 8u of the row, codes at bit 16g + 8u
#pragma unroll
        for (int b = R0; b < R1; ++b) {
            const uint32_t code = F.idx[b] >> (16 * (g & 1));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const u32x4 e = expand_two_groups(uint2{F.a[b][2 * u], F.a[b][2 * u + 1]}, (code >> (8 * u)) & 0xFFu);
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    acc[4 * h + b][bj] = mfma_dense<T>(e, u ? hi4(B[bj]) : lo4(B[bj]), acc[4 * h + b][bj]);
            }
        }
    }
}

// Order barrier between the parts of a half (the compiler keeps program order across it).
__device__ __forceinline__ void part_fence() { __builtin_amdgcn_sched_barrier(0); }

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Weight slice of the block in registers on its way to LDS: a wave's share (4 x 1 KiB of a dense
// slice; 2 x 1 KiB of 2:4 values and its code words of a 2:4 slice).
struct WRegs {
    u32x4 w[4];
    uint32_t m[2];
};

// Per-lane sources and LDS slots of a wave's share of each weight slice.  The LDS image of a slice
// is that of the LDS-staged kernel: 64-row groups 8 KiB apart, a dense group as 8 kilobytes (packed:
// kilobyte j % 2 of 16-row panel j / 2, the stored order; row-major W: rows of XOR-swizzled
// chunks), a 2:4 group as 4 kilobytes of stored values (panel j), then the code words of both
// groups, row-major per group.
template <int BK, bool HYB, int ES>
struct WCopy {
    static constexpr int KSL = slice_k<ES>(), MGB = meta_group_bytes<ES>(), WPR = KSL / 32;
    static constexpr int NCW = 2 * MGB / 1024;   // code words per lane and slice (both groups)
    rsrc_t wr, mr;                 // values (or W rows) and codes of the tile row from its first tile
    uint32_t vbase, mbase;         // first value / code word of the tile row
    int64_t ldw;
    uint32_t dvo[2];               // dense job w + 4v of a group: per-lane source offset
    uint32_t svo;                  // 2:4 values job w of a group
    uint32_t mvo[NCW];             // code word 256 v + 64 w + lane of the slice: per-lane source offset
    int wave, lane;

    // global -> registers: slice kn (its tile's value / code offsets voff, moff).  The same six load
    // instructions whatever the type -- a 2:4 slice repeats its value loads and a dense one loads a
    // code word it does not store -- so no register is defined differently on two paths (which
    // would make the compiler copy them, and wait for the loads to do so).
    __device__ __forceinline__ void load(WRegs& R, bool dense, uint32_t voff, uint32_t moff, int kn) const {
        const int s = kn % (BK / KSL);
        if (!HYB) {
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
#pragma unroll
                for (int v = 0; v < 2; ++v)
                    R.w[2 * gi + v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        wr, dvo[v], (uint32_t)(ES * 64 * gi * ldw + 128 * (int64_t)kn), 0));
            return;
        }
        const uint32_t so_d = ES * (voff - vbase) + 2048 * s, so_s = ES * (voff - vbase) + 1024 * s;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                // dense: job w + 4v of group gi; 2:4: the values job w of group gi (loaded twice)
                const uint32_t vo = dense ? dvo[v] : svo;
                const uint32_t so = dense ? so_d + ES * 64 * gi * BK : so_s + ES * 64 * gi * (BK / 2);
                R.w[2 * gi + v] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, vo, so, 0));
            }
        const uint32_t som = 4 * (moff - mbase + WPR * s);   // past the codes for a late dense tile: reads 0
#pragma unroll
        for (int v = 0; v < 2; ++v)
            R.m[v] = __builtin_amdgcn_raw_buffer_load_b32(mr, mvo[v < NCW ? v : 0], som, 0);
    }
    // registers -> the LDS stage `st` (sink: 2 KiB nobody reads).  The same six writes whatever the
    // type: a 2:4 slice sends its repeated value loads, a dense one its code words, to the sink --
    // no branch, so the writes can be interleaved with the products of the same block.
    __device__ __forceinline__ void store(const WRegs& R, bool dense, uint8_t* st, uint8_t* sink) const {
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                uint8_t* d = st + gi * kGroupBytes + 1024 * (wave + 4 * v) + 16 * lane;   // dense job
                if (HYB) {
                    uint8_t* sp = v == 0 ? st + gi * kGroupBytes + 1024 * wave + 16 * lane : sink + 1024 * gi + 16 * lane;
                    d = dense ? d : sp;
                }
                st16(d, R.w[2 * gi + v]);
            }
        if (HYB) {
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                uint8_t* d = (dense || v >= NCW) ? sink + 4 * (64 * v + lane)
                                                 : st + 2 * kGroupBytes + 4 * (256 * v + 64 * wave + lane);
                *reinterpret_cast<uint32_t*>(d) = R.m[v];
            }
        }
    }
};

template <typename T, int BK, bool HYB, int SP>
__global__ __launch_bounds__(256) void gemm_prefill_xr_kernel(const GemmArgs a, int NB, int MB, int ord, int lch) {
    constexpr int ES = Elem<T>::bytes, KSL = slice_k<ES>(), MGB = meta_group_bytes<ES>();
    constexpr int BN = 128, BMX = 256, NW = 4, SPT = BK / KSL;
    using Lo = Layout<BN, 0, 3, MGB>;          // three LDS stages of the weight slice
    static_assert(Lo::WOFF == 0 && Lo::MOFF == 2 * kGroupBytes, "stage layout");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int nb, mb;
    block_of(blockIdx.x, NB, MB, ord, nb, mb);
    const int64_t n0 = (int64_t)nb * BN, m0 = (int64_t)mb * BMX;
    const int Tk = (int)(a.K / BK);

    // the ordered tile list (the copy-job fields of Ctx are not used here)
    Ctx<BK, HYB, BN, 0, NW> C;
    C.n0 = n0;
    C.Tk = Tk;
    if (HYB) {
        load_tile_list<Lo>(C, a, lch, tid, lane);
    } else {
        C.lnd = 0u;
#pragma unroll
        for (int w = 0; w < 4; ++w) C.lv[w] = C.lm[w] = C.lc[w] = 0u;
    }

    WCopy<BK, HYB, ES> WC;
    WC.wave = wave;
    WC.lane = lane;
    WC.ldw = a.ldw;
    {
        const uint8_t* Vb = reinterpret_cast<const uint8_t*>(a.values);
        const uint8_t* Wb = reinterpret_cast<const uint8_t*>(a.W);
        if (HYB) {
            const hts_tile first = a.index[(n0 / a.bn) * Tk];
            WC.vbase = first.val_off;
            WC.mbase = first.meta_off;
            WC.wr = make_rsrc(Vb + (uint64_t)ES * WC.vbase, (uint64_t)Tk * BN * BK * ES);
            WC.mr = make_rsrc(a.meta + WC.mbase, (uint64_t)Tk * BN * BK / 8);
        } else {
            // rows past N (N is a multiple of 64) read zeros and feed only unstored outputs
            WC.vbase = WC.mbase = 0;
            WC.wr = make_rsrc(Wb + ES * n0 * a.ldw, (uint64_t)(a.N - n0) * a.ldw * ES);
            WC.mr = WC.wr;
        }
#pragma unroll
        for (int v = 0; v < 2; ++v) {
            const int job = wave + 4 * v;
            const int row = 8 * job + (lane >> 3), col = (lane & 7) ^ ((row >> 1) & 7);
            WC.dvo[v] = HYB ? (uint32_t)((job >> 1) * 16 * BK * ES + 1024 * (job & 1) + 16 * lane)
                            : (uint32_t)(ES * (int64_t)row * a.ldw + 16 * col);
        }
        WC.svo = (uint32_t)(wave * 16 * (BK / 2) * ES + 16 * lane);
        constexpr int WPR = KSL / 32;
#pragma unroll
        for (int v = 0; v < WCopy<BK, HYB, ES>::NCW; ++v) {
            const int wi = 256 * v + 64 * wave + lane;                 // word of the slice's codes image
            const int gi = wi / (64 * WPR), rr = (wi % (64 * WPR)) / WPR, wd = wi % WPR;
            WC.mvo[v] = (uint32_t)(4 * ((64 * gi + rr) * (BK / 32) + wd));
        }
    }

    // X: this wave's four 16-row panels of the block, from the panel copy of X (xpanel)
    const int i = lane & 15, g = lane >> 4;
    const int64_t xrow0 = m0 + 64 * wave;
    const int64_t pstride = 16 * a.K * ES;                          // bytes per 16-row panel
    const int64_t npanel = (a.M + 15) / 16, p0 = xrow0 / 16;
    const rsrc_t xr = make_rsrc(reinterpret_cast<const uint8_t*>(a.xpanel) + p0 * pstride,
                                p0 < npanel ? (uint64_t)(npanel - p0) * pstride : 0ull);
    uint32_t xv[4];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
        xv[bj] = (uint32_t)(bj * pstride + (SP == SPARSE_SMFMAC ? 16 * lane : 512 * g + 16 * i));

    f32x4 acc[8][4];
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) acc[b][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int S = Tk * SPT, lcs = lch + (SPT == 2 ? 1 : 0);   // slices per chunk: 2^lcs
    // slice kn is dense when it lies in the dense run at the start of its chunk (chunk-ordered list)
    auto dense_slice = [&](int kn) __attribute__((always_inline)) {
        return !HYB || (kn & ((1 << lcs) - 1)) < SPT * (int)__builtin_amdgcn_readlane((int)C.lnd, kn >> lcs);
    };
    // Loads past the last slice are issued anyway, of the last slice again: every path then issues
    // the same loads, so the compiler's count of outstanding loads (and the waits it derives for the
    // operands) is exact at every join instead of assuming the shortest path.
    uint32_t xlc[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) xlc[w] = C.lc[w];
    auto load_w = [&](WRegs& R, int kn) __attribute__((always_inline)) {     // called with kn = 0, 1, 2, ...
        if (HYB && kn < S && kn > 0 && kn % (64 * SPT) == 0) C.shift_list();
        const int kc = kn < S ? kn : S - 1;
        const int p = kc / SPT;
        const uint32_t voff = HYB ? list_entry(C.lv, p) : 0u, moff = HYB ? list_entry(C.lm, p) : 0u;
        WC.load(R, dense_slice(kc), voff, moff, kc);
    };
    auto load_x = [&](u32x8 (&B)[4], int kn) __attribute__((always_inline)) {   // called with kn = 0, 1, 2, ...
        if (HYB && kn < S && kn > 0 && kn % (64 * SPT) == 0) {
#pragma unroll
            for (int w = 0; w < 3; ++w) xlc[w] = xlc[w + 1];
            xlc[3] = 0u;
        }
        const int kc = kn < S ? kn : S - 1;
        const int p = kc / SPT, s = kc % SPT;
        const int tk = HYB ? (int)__builtin_amdgcn_readlane((int)xlc[0], p & 63) : p;
        load_xr<SP>(B, xr, xv, (uint32_t)(16 * (ES * tk * BK + 128 * s)));   // chunk column * 256 bytes
    };
    auto stage = [&](int kn) __attribute__((always_inline)) { return smem + (kn % 3) * Lo::STAGE; };

    // prologue: W(0), W(1) into stages 0 and 1, W(2) and X(0) in flight, half 0 of slice 0 read
    // register sets rotate with the slice: P = ks % 3 -- X(ks) in B[P] (loaded two slices ahead),
    // W(ks+3) loaded into R[P], W(ks+2) (loaded one slice ago, in R[(P+2) % 3]) written to LDS
    WRegs R[3];
    u32x8 B[3][4];
    Frags H0, H1;
    load_w(R[0], 0);
    load_x(B[0], 0);
    load_w(R[1], 1);
    load_x(B[1], 1);
    WC.store(R[0], dense_slice(0), stage(0), smem + Lo::SINK);
    WC.store(R[1], dense_slice(S > 1 ? 1 : 0), stage(1), smem + Lo::SINK);
    load_w(R[2], 2);
    barrier_lds();
    read_half<T, SP, HYB, 0>(H0, stage(0), dense_slice(0), lane);

    // slice ks (B and R register sets P = ks % 2; weight stage ks % 3): barrier -- stage ks+1
    // complete, stage ks+2 no longer read; first half: products of half 0 while half 1 of slice ks
    // is read and the X(ks+1) and W(ks+3) loads issue; second half: products of half 1 while half 0
    // of slice ks+1 is read and W(ks+2) is written to its stage
    auto slice = [&](auto PP, auto DD, int ks) __attribute__((always_inline)) {
        constexpr int P = decltype(PP)::value;
        constexpr bool DENSE = decltype(DD)::value;
        barrier_lds();
        const int kn1 = ks + 1 < S ? ks + 1 : S - 1;
        const bool next_dense = dense_slice(kn1);
        // rows of a half: dense 8 (32 products), 2:4 4 (16)
        constexpr int RH = DENSE ? 8 : 4, Q = RH / 4;
        // first half: products of half 0 (fragments read in the previous slice), with the reads of
        // half 1 and the global loads of later slices issued among them
        read_half<T, SP, HYB, 1>(H1, stage(ks), DENSE, lane);
        part_fence();
        mma_part<T, SP, DENSE, 0, 0, Q>(acc, H0, B[P], lane);
        part_fence();
        load_x(B[(P + 2) % 3], ks + 2);
        part_fence();
        mma_part<T, SP, DENSE, 0, Q, 2 * Q>(acc, H0, B[P], lane);
        part_fence();
        load_w(R[P], ks + 3);
        part_fence();
        mma_part<T, SP, DENSE, 0, 2 * Q, RH>(acc, H0, B[P], lane);
        part_fence();
        wait_lgkm0();                        // half 1 has long landed: no later wait counts these reads
        // second half: products of half 1, with the reads of half 0 of slice ks+1 and the weight
        // writes of slice ks+2 among them
        mma_part<T, SP, DENSE, 1, 0, Q>(acc, H1, B[P], lane);
        part_fence();
        read_half<T, SP, HYB, 0>(H0, stage(ks + 1), next_dense, lane);
        part_fence();
        mma_part<T, SP, DENSE, 1, Q, 3 * Q>(acc, H1, B[P], lane);
        part_fence();
        WC.store(R[(P + 2) % 3], dense_slice(ks + 2 < S ? ks + 2 : S - 1), stage(ks + 2), smem + Lo::SINK);
        part_fence();
        mma_part<T, SP, DENSE, 1, 3 * Q, RH>(acc, H1, B[P], lane);
        part_fence();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // slices ks .. end-1, all of one type: the register sets follow ks % 3, so the unrolled triples
    // start on a multiple of three
    using I2 = std::integral_constant<int, 2>;
    auto run = [&](int& ks, int end, auto DD) __attribute__((always_inline)) {
        if (ks < end && ks % 3 == 1) slice(I1{}, DD, ks++);
        if (ks < end && ks % 3 == 2) slice(I2{}, DD, ks++);
        for (; ks + 2 < end; ks += 3) {
            slice(I0{}, DD, ks);
            slice(I1{}, DD, ks + 1);
            slice(I2{}, DD, ks + 2);
        }
        if (ks < end) slice(I0{}, DD, ks++);
        if (ks < end) slice(I1{}, DD, ks++);
    };
    using DenseT = std::true_type;
    using SparseT = std::false_type;
    int ks = 0;
    if constexpr (!HYB) {
        run(ks, S, DenseT{});
    } else {
        // chunk by chunk: its dense run, then its 2:4 run
        while (ks < S) {
            const int c = ks >> lcs, cs = c << lcs;
            const int ce = (cs + (1 << lcs)) < S ? cs + (1 << lcs) : S;
            int de = cs + SPT * (int)__builtin_amdgcn_readlane((int)C.lnd, c);
            de = de < ce ? de : ce;
            run(ks, de, DenseT{});
            run(ks, ce, SparseT{});
        }
    }

    // epilogue: acc[b][bj] lane (j + 16q) holds Y^T rows 4q..4q+3 of block b, column j of block bj
    const int j = lane & 15, q = lane >> 4;
    if (a.gate) {
        // every gate value of the lane is loaded before the first store, since G may be Y
        f32x4 gv[8][4];
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t m = xrow0 + 16 * bj + j, n = n0 + 16 * b + 4 * q;
                gv[b][bj] = (m < a.M && n < a.N) ? load_gate4(a.gate, m * a.ldg + n, a.y_dtype)
                                                 : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int b = 0; b < 8; ++b)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) acc[b][bj] = silu_times4(gv[b][bj], acc[b][bj]);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int64_t n = n0 + 16 * b + 4 * q;
        if (n >= a.N) continue;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t m = xrow0 + 16 * bj + j;
            if (m < a.M) store_y4(a.Y, m * a.ldy + n, a.y_dtype, acc[b][bj]);
        }
    }
}

// X[M,K] rearranged into 16-row panels: chunk c (16 bytes) of panel row j at (16 c + j) * 16 bytes
// from the panel start, rows past M zero.  One chunk per thread, consecutive threads on consecutive
// destination chunks (whole cache lines written).
__global__ __launch_bounds__(256) void pack_xpanel_kernel(const uint8_t* __restrict__ X, int64_t ldxb, int64_t M,
                                                          int64_t cpr, uint8_t* __restrict__ P, int64_t total) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int64_t p = t / (16 * cpr), rem = t - p * 16 * cpr, c = rem >> 4, j = rem & 15;
    const int64_t row = 16 * p + j;
    const u32x4 v = row < M ? ld16(X + row * ldxb + 16 * c) : u32x4{0u, 0u, 0u, 0u};
    st16(P + 16 * t, v);
}

// Workgroup order: each XCD a contiguous range, groups of 4 N-blocks, N fastest (the 32 workgroups
// an XCD runs together then cover 4 tile rows x 8 blocks of 256 X rows).  HTS_PREFILL_XR_ORDER
// overrides (code as for the LDS-staged kernel's order).
int prefill_xr_order() {
    const char* e = getenv("HTS_PREFILL_XR_ORDER");
    const int v = (e && *e) ? atoi(e) : -1;
    const int g = (v >> 1) & 31;
    if (v < 0 || v > 127 || g == 0) return 1 | (4 << 1);
    return v;
}

template <typename T, int BK, bool HYB, int SP>
hipError_t launch_xr(const GemmArgs& a, hipStream_t s) {
    using Lo = Layout<128, 0, 3, meta_group_bytes<Elem<T>::bytes>()>;
    auto kern = gemm_prefill_xr_kernel<T, BK, HYB, SP>;
    static DeviceOnce lds_limit;   // per instantiation and device
    hipError_t e = lds_limit.run([&] {
        return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Lo::TOTAL);
    });
    if (e != hipSuccess) return e;
    // X into 16-row panels (the caller's workspace), then the product
    constexpr int ES = Elem<T>::bytes;
    const int64_t cpr = a.K * ES / 16, total = ((a.M + 15) / 16) * 16 * cpr;
    pack_xpanel_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(
        reinterpret_cast<const uint8_t*>(a.X), a.ldx * ES, a.M, cpr, static_cast<uint8_t*>(a.xpanel), total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int NB = (int)((a.N + 127) / 128), MB = (int)((a.M + 255) / 256);
    kern<<<dim3((unsigned)(NB * MB)), dim3(256), Lo::TOTAL, s>>>(a, NB, MB, prefill_xr_order(), prefill_chunk_log2(BK));
    return hipGetLastError();
}

template <typename T, int BK, bool HYB>
hipError_t launch_xr_sp(const GemmArgs& a, int sp, hipStream_t s) {
    if constexpr (Elem<T>::bytes == 1) {
        (void)sp;
        return launch_xr<T, BK, HYB, SPARSE_SMFMAC>(a, s);   // 8-bit: no expansion path
    } else {
        return sp == SPARSE_SMFMAC ? launch_xr<T, BK, HYB, SPARSE_SMFMAC>(a, s)
                                   : launch_xr<T, BK, HYB, SPARSE_DECOMPRESS>(a, s);
    }
}

template <typename T>
hipError_t launch_xr_bk(const GemmArgs& a, int sp, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128) return hyb ? launch_xr_sp<T, 128, true>(a, sp, s) : launch_xr_sp<T, 128, false>(a, sp, s);
    return hyb ? launch_xr_sp<T, 64, true>(a, sp, s) : launch_xr_sp<T, 64, false>(a, sp, s);
}

}  // namespace

// HTS_PREFILL_KERNEL=xr sends every unsplit product on 128-row tiles (or a row-major W) with X
// panels in the workspace here; otherwise (default, or =lds) the LDS-staged kernel runs.
bool prefill_xr_wanted(int64_t M, int32_t bn, bool packed) {
    (void)M;
    const char* e = getenv("HTS_PREFILL_KERNEL");
    if (!(e && !strcmp(e, "xr"))) return false;
    return !packed || bn == 128;
}

bool prefill_xr_applies(const GemmArgs& a) {
    return a.xpanel != nullptr && a.nsplit <= 1 && prefill_xr_wanted(a.M, a.bn, a.index != nullptr);
}

hipError_t launch_gemm_prefill_xr(const GemmArgs& a, int sparse_path, hipStream_t s) {
    if (a.dtype == HTS_FP8_E4M3)   // 128x128 tiles only
        return a.index ? launch_xr_sp<FP8T, 128, true>(a, sparse_path, s)
                       : launch_xr_sp<FP8T, 128, false>(a, sparse_path, s);
    return a.dtype == HTS_BF16 ? launch_xr_bk<BF16T>(a, sparse_path, s) : launch_xr_bk<F16T>(a, sparse_path, s);
}

}  // namespace hts
