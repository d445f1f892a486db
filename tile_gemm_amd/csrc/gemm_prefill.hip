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
// N-blocks (11 for 8-bit data; N fastest inside a group): blocks running together
// on one XCD share their W and X slices in its L2.
#include <cstring>

#include "prefill_common.h"

namespace hts {
namespace {

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
    if constexpr (Elem<T>::bytes == 1) {
        // 8-bit: both chunks of a row block form one 16x16x128 operand (one instruction per block)
        u32x4 A[2][NBI];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int b = 0; b < NBI; ++b) A[u][b] = ld16(ws + b * 2048 + (u ? a1 : a0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < NBI; ++b)
#pragma unroll
            for (int bj = 0; bj < NBJ; ++bj) acc[b][bj] = mfma_fp8_dense128(cat8(A[0][b], A[1][b]), Bx[bj], acc[b][bj]);
        return;
    }
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

// ms: the group's codes, code row by code row (BK/32 words per row: every slice of the tile); s:
// the slice of the tile.
template <typename T, int BK, int SP, int NBI, int NBJ>
__device__ __forceinline__ void compute_sparse(f32x4 (&acc)[NBI][NBJ], const uint8_t* xs, const uint8_t* ws,
                                               const uint32_t* ms, int s, int lane) {
    constexpr int CPR = BK / 32;            // code words per row in LDS
    const int cs = (128 / (32 * Elem<T>::bytes)) * s;   // first word of slice s in a row (16-bit: 2 s)
    const int i = lane & 15, g = lane >> 4;
    const int s0 = 16 * (16 * g + i);    // stored order: chunk g of row i of the 16-row block
    u32x8 Bx[NBJ];
    load_x<SP, NBJ>(Bx, xs, lane);
#pragma unroll
    for (int h = 0; h < NBI / 4; ++h) {
        const uint8_t* wg = ws + h * kGroupBytes;
        const uint32_t* mg = ms + h * (kGroupBytes / 4);   // each group's codes sit in its own slot
        if (SP == SPARSE_SMFMAC) {
            u32x4 A[4];
            uint32_t idx[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                A[b] = ld16(wg + b * 1024 + s0);
                // 16-bit: a 16-bit half of the row's word g/2; 8-bit: the row's whole word g
                idx[b] = Elem<T>::bytes == 1 ? mg[CPR * (16 * b + i) + cs + g]
                                             : mg[CPR * (16 * b + i) + cs + (g >> 1)] >> (16 * (g & 1));
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
                    const uint32_t code = (mg[CPR * (16 * b + i) + cs + (g >> 1)] >> (16 * (g & 1) + 8 * u)) & 0xFFu;
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

// Wait until the oldest slice in flight has landed, leaving min(NSTAGE - 2, later) younger
// slices in flight (`later` = slices issued after it); each slice is PER copies per wave.
template <int NSTAGE, int PER>
__device__ __forceinline__ void wait_slice(int later) {
    const int k = later < NSTAGE - 2 ? later : NSTAGE - 2;
    if (NSTAGE >= 4 && k >= 2) wait_vm<(NSTAGE >= 4 ? 2 * PER : 0)>();
    else if (NSTAGE >= 3 && k >= 1) wait_vm<(NSTAGE >= 3 ? PER : 0)>();
    else wait_vm<0>();
}

// TWO: the block covers two 64-row tile rows (64-row tiles, 16-bit data); it walks K in tile-column
// order and each wave feeds its own row's tile to the matrix cores by that tile's type.  Its
// per-slice choices of copy source cost registers: it is held to two waves per SIMD (two
// workgroups per CU), which the 128 x 64 and 128 x 128 forms reach without spills.
template <typename T, int BK, bool HYB, int SP, int BN, int BM, int NSTAGE, int NW, bool TWO = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(TWO ? 2 : 1)))
void gemm_prefill_kernel(const GemmArgs a, int NB, int MB, int ord, int lch) {
    constexpr int ES = Elem<T>::bytes, KSL = slice_k<ES>(), MGB = meta_group_bytes<ES>();
    using Lo = Layout<BN, BM, NSTAGE, MGB>;
    static_assert(NW == 4 || NW == 8, "4 or 8 waves");
    static_assert(!TWO || (HYB && BN == 128 && NSTAGE == 2 && ES == 2 && NW == 4), "two 64-row tile rows");
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
        // a group's codes: one job, lane L the 16 bytes of code row L (issue_codes)
        C.mvo = (uint32_t)(16 * lane);
    }
    // ordered tile list of the tile row, tile columns kept for the X copies
    SecondRow R2;                  // blocks of two tile rows only
    if constexpr (TWO) {
        load_two_lists<Lo>(C, R2, a, tid, lane);
    } else if (HYB) {
        load_tile_list<Lo>(C, a, lch, tid, lane);
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
        for (int b = 0; b < k0 / (64 * SPT); ++b) {
            C.shift_list();
            if constexpr (TWO) R2.shift();
        }
    auto issue = [&](int kn) {   // called for kn = k0, k0 + 1, ... in order
        if (HYB && kn > k0 && kn % (64 * SPT) == 0) {
            C.shift_list();
            if constexpr (TWO) R2.shift();
        }
        const uint32_t stage = (kn % NSTAGE) * Lo::STAGE;
        if constexpr (TWO) {
            C.xso = (uint32_t)(ES * (kn / SPT) * BK + 128 * (kn % SPT));   // tile column in K order
            issue_slice_two(C, R2, kn, stage);
            return;
        }
        set_x(kn);
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
    } else if constexpr (TWO) {
        // K order; the type of this wave's tile is read before step() issues the next slice (which
        // may move the list registers on to the next 64 tile columns)
        for (; ks < k1; ++ks) {
            const bool sparse = (list_entry(C.lc, ks / SPT) >> wn) & 1u;
            const uint8_t* st = step(ks);
            if (!wvalid) continue;
            const uint8_t* ws = st + Lo::WOFF + wn * kGroupBytes;
            if (sparse)
                compute_sparse<T, BK, SP, 4, NBJ>(acc, st + xoff, ws, reinterpret_cast<const uint32_t*>(ws + Lo::MHALF),
                                                  ks % SPT, lane);
            else
                compute_dense<T, SP, 4, NBJ, true>(acc, st + xoff, ws, lane);
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
                    compute_sparse<T, BK, SP, 4, NBJ>(acc, st + xoff, st + Lo::WOFF + wn * kGroupBytes,
                                                      reinterpret_cast<const uint32_t*>(st + Lo::WOFF + wn * kGroupBytes + Lo::MHALF),
                                                      ks % SPT, lane);
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

// Block order of the tiled kernels (HTS_PREFILL_ORDER overrides; see block_of): contiguous per XCD,
// N fastest, in groups of 8 N-blocks for 16-bit data and 11 for 8-bit data.  Interleaved sweeps of
// 6 to 16 N-blocks per group on two boxes: the 8-bit 7B up-projection at M = 2048 ran 1.05x faster
// with 11 on both; on the 16-bit layers (7B up, gate and down, 13B, the 4096^2 sweep) no group
// size won everywhere (0.96-1.05x, box to box), so they keep 8.
int prefill_order(int elem_bytes) {
    const char* e = getenv("HTS_PREFILL_ORDER");
    const int v = (e && *e) ? atoi(e) : -1;
    const int g = (v >> 1) & 31;
    if (v < 0 || v > 127 || g == 0)   // groups of at least one N-block
        return 1 | ((elem_bytes == 1 ? kGroupN8 : kGroupN) << 1);
    return v;
}

template <typename T, int BK, bool HYB, int SP, int BN, int BM, int NSTAGE, int NW = 4, bool TWO = false>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    using Lo = Layout<BN, BM, NSTAGE, meta_group_bytes<Elem<T>::bytes>()>;
    auto kern = gemm_prefill_kernel<T, BK, HYB, SP, BN, BM, NSTAGE, NW, TWO>;
    // one flag set per instantiation (this static) and device
    static DeviceOnce lds_limit;
    hipError_t e = lds_limit.run([&] {
        return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Lo::TOTAL);
    });
    if (e != hipSuccess) return e;
    const int NB = (int)((a.N + BN - 1) / BN), MB = (int)((a.M + BM - 1) / BM);
    const int nsplit = a.nsplit > 1 ? a.nsplit : 1;
    kern<<<dim3((unsigned)(NB * MB), (unsigned)nsplit), dim3(64 * NW), Lo::TOTAL, s>>>(a, NB, MB, prefill_order(Elem<T>::bytes),
                                                                                   prefill_chunk_log2(BK));
    e = hipGetLastError();
    if (e != hipSuccess || nsplit == 1) return e;
    const int64_t quads = a.M * (a.N / 4);
    split_sum_kernel<<<dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s>>>(a.part, nsplit, a.gate, a.ldg, a.M, a.N, a.Y,
                                                                              a.ldy, a.y_dtype);
    return hipGetLastError();
}

template <typename T, int BK, bool HYB, int SP>
hipError_t launch4(const GemmArgs& a, hipStream_t s) {
    // 128 weight rows (one tile row, or two of 64-row tiles) x 128 (or 64 or 192, prefill_block_m)
    // X rows per workgroup, 4 waves, 2 stages (two workgroups per CU)
    if constexpr (Elem<T>::bytes == 1) {
        if (prefill_block_m(a.M, a.N, a.dtype, 128) == 192) return launch_tile<T, BK, HYB, SP, 128, 192, 2>(a, s);
        return launch_tile<T, BK, HYB, SP, 128, 128, 2>(a, s);
    } else {
        if constexpr (HYB) {
            // 64-row tiles: two tile rows per block, 64 or 128 X rows (192 would need more than the
            // 256 registers that let two workgroups share a CU)
            if (a.bn == 64 && prefill_weight_rows(64) == 128) {
                if (prefill_block_m(a.M, a.N, a.dtype, 128) == 64) return launch_tile<T, BK, HYB, SP, 128, 64, 2, 4, true>(a, s);
                return launch_tile<T, BK, HYB, SP, 128, 128, 2, 4, true>(a, s);
            }
        }
        const int bm = prefill_block_m(a.M, a.N, a.dtype, (HYB && a.bn == 64) ? 64 : 128);
        if (bm == 64) {
            if (HYB && a.bn == 64) return launch_tile<T, BK, HYB, SP, 64, 64, 2>(a, s);
            return launch_tile<T, BK, HYB, SP, 128, 64, 2>(a, s);
        }
        if (HYB && a.bn == 64) return launch_tile<T, BK, HYB, SP, 64, 128, 2>(a, s);
        if (bm == 192) return launch_tile<T, BK, HYB, SP, 128, 192, 2>(a, s);
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

// Tile columns per chunk of the ordered list, as log2: chunks of 512 K by default
// (HTS_PREFILL_CHUNK = 4, 8, 16, 32 or 64 tile columns overrides).
int prefill_chunk_log2(int bk) {
    const char* e = getenv("HTS_PREFILL_CHUNK");
    const int v = (e && *e) ? atoi(e) : 512 / bk;
    for (int l = 2; l <= 6; ++l)
        if (v == (1 << l)) return l;
    return bk == 64 ? 3 : 2;
}

// X rows per block (block_rows: weight rows per block, 128 or 64).
//  - 64 for 16-bit data at M <= 64, where a 128-row block would copy (and multiply) at least half
//    padding rows.  Interleaved A/B, 64 against 128 rows: M = 33 .. 64 on the 7B, 13B and block
//    layers 1.00-1.04x (bit-identical results); M = 96 .. 512 0.65-1.06x, mostly slower (each
//    weight slice is then copied once per 64 X rows).
//  - 192 or 128 above.  A 128 x 192 block copies 40 KiB per 64-wide slice for 1.5x the products of
//    a 128 x 128 block (32 KiB), and the copies set the pace: it takes about 1.39x as long.  The
//    grid runs in rounds of 512 blocks (two per CU) and a partial last round costs nearly a whole
//    one, so 192 rows are taken when their rounds x 1.39 undercut the 128-row rounds by 3%.
//    Dense product, interleaved, 128 / 192 rows, us: 7B up M = 2048 189.9 / 175.6 (3 / 2 rounds),
//    M = 4096 351.5 / 331.3 (6 / 4), 13B 5120^2 M = 4096 214.6 / 207.8 (3 / 2), 13B up M = 4096
//    528.9 / 521.7 (7 / 5: within the margin, 128 kept); 4096^2 M = 2048 70.6 / 87.9 and 7B up
//    M = 1024 114.8 / 128.8 (same rounds: 128 kept).  8-bit hybrid (its slices are also 128 bytes
//    of each row): 7B up M = 2048 100.9 / 92.3, M = 4096 182.5 / 169.2, M = 1024 58.5 / 69.4.
//  8-bit data never takes 64 rows.
// HTS_PREFILL_BLOCK_M = 64 (16-bit), 128 or 192 (128-row weight blocks) overrides.
int prefill_block_m(int64_t M, int64_t N, int32_t dtype, int block_rows) {
    const bool fp8 = dtype == HTS_FP8_E4M3;
    const char* v = getenv("HTS_PREFILL_BLOCK_M");
    if (v && !strcmp(v, "64") && !fp8) return 64;
    if (v && !strcmp(v, "128")) return 128;
    if (v && !strcmp(v, "192")) return block_rows == 128 ? 192 : 128;
    if (M <= 64) return fp8 ? 128 : 64;
    if (block_rows != 128) return 128;
    const int64_t nb = (N + 127) / 128;
    const int64_t b128 = nb * ((M + 127) / 128), b192 = nb * ((M + 191) / 192);
    if (b128 <= 256) return 128;                  // split products: the planner fills the chip
    const int64_t r128 = (b128 + 511) / 512, r192 = (b192 + 511) / 512;
    return r192 * 139 < r128 * 97 ? 192 : 128;
}

// Weight rows per block of a packed weight with bn-row tiles (16-bit data): 128, so 64-row tiles
// go two tile rows to a block (HTS_PREFILL_TWO_ROWS=0: one 64-row tile row per block instead).
int prefill_weight_rows(int bn) {
    if (bn != 64) return 128;
    const char* v = getenv("HTS_PREFILL_TWO_ROWS");
    return (v && !strcmp(v, "0")) ? 64 : 128;
}

hipError_t launch_gemm_prefill(const GemmArgs& a, int sparse_path, hipStream_t s) {
    if (a.dtype == HTS_FP8_E4M3)   // 128x128 tiles only
        return a.index ? launch3<FP8T, 128, true>(a, sparse_path, s) : launch3<FP8T, 128, false>(a, sparse_path, s);
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, sparse_path, s) : launch2<F16T>(a, sparse_path, s);
}

}  // namespace hts
