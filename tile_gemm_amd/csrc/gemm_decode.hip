// Hybrid tile-sparse product for small M (M <= 16; M <= 32 on 128-wide tiles,
// where each weight fragment feeds two groups of 16 X rows): the HBM-streaming path.
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
#include <cstdlib>

#include "gemm_common.h"

namespace hts {
namespace {

// Packed weight loads: every weight byte is read once, in whole kilobytes per instruction, so they
// are marked non-temporal (streaming) and leave the caches to X and the index records, which every
// workgroup re-reads.  Measured on the 7B up-projection: M=1 16.5 -> 14.5 us, M=16 19.7 -> 18.1 us
// (bf16); M=1 10.3 -> 9.3 us (8-bit).  Row-major weights keep ordinary loads: a 16-byte-per-lane
// load there uses half of each cache line it touches, and the other half is read by a later load
// (non-temporal: 17.7 -> 19.0 us at M=1).  Pack and unpack were slower with non-temporal access too.
__device__ __forceinline__ u32x4 ldw16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Lanes of one wave exchange data through that wave's own LDS (X staging, partial sums).  The LDS
// operations of a wave execute in issue order, so no wait is needed between a write and a read of
// another lane's slot; this keeps the compiler from moving LDS accesses across the exchange
// (release and acquire fences at wavefront scope around a wave barrier emit no instructions).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int BK, int PP, int MG = 1>
struct TileRegs {
    u32x4 a[PP][BK / 32];      // per panel: dense: BK/32 chunks; 2:4: BK/64 chunks
    uint32_t m[PP][BK / 64];   // per panel: 2:4 metadata words, one per slice
    u32x4 x[MG][BK / 32];      // X chunks of MG groups of 16 rows, shared by the PP panels
};

// Loads of tile column tk for PP consecutive 16-row panels (rows n0 .. n0 + 16 PP - 1, all in
// one tile row: r0 + 16 PP <= bn) and the matching X chunks.
template <typename T, int BK, bool HYB, int SP, int PP, bool XT, int MG>
__device__ __forceinline__ uint32_t load_tile(TileRegs<BK, PP, MG>& R, const GemmArgs& a, const hts_tile& e, int tk,
                                              int64_t n0, int r0, int lane, const uint16_t* xrow) {
    static_assert(MG == 1 || XT, "two X row groups are loaded as whole rows");
    const int i = lane & 15, g = lane >> 4;
    uint32_t type = HTS_TILE_DENSE;
    uint32_t moff = 0;
    if (HYB) {
        type = e.type;
        moff = e.meta_off;
    }
    if (!HYB) {        // row-major W: lane i reads row i
        const uint16_t* base = a.W + (n0 + i) * a.ldw + (int64_t)tk * BK;
#pragma unroll
        for (int q = 0; q < PP; ++q)
#pragma unroll
            for (int u = 0; u < BK / 32; ++u) R.a[q][u] = ld16(base + 16 * q * a.ldw + koff<SP>(u, g));
    } else if (type == HTS_TILE_DENSE) {
        // packed tile: 16-row panels of BK-element rows, chunk c of panel row i at (16 c + i) chunks
        // from the panel start -- the four chunks of a substep are one contiguous kilobyte
        const uint16_t* panel = a.values + e.val_off + (int64_t)r0 * BK;
#pragma unroll
        for (int q = 0; q < PP; ++q)
#pragma unroll
            for (int u = 0; u < BK / 32; ++u) R.a[q][u] = ldw16(panel + 16 * q * BK + (16 * (koff<SP>(u, g) / 8) + i) * 8);
    } else {
        const uint32_t* mrow = a.meta + moff + (int64_t)(r0 + i) * (BK / 32);
        const uint16_t* panel = a.values + e.val_off + (int64_t)r0 * (BK / 2);   // stored rows: BK/2 values
#pragma unroll
        for (int q = 0; q < PP; ++q)
#pragma unroll
            for (int s = 0; s < BK / 64; ++s) R.a[q][s] = ldw16(panel + 16 * q * (BK / 2) + (16 * (4 * s + g) + i) * 8);
#pragma unroll
        for (int q = 0; q < PP; ++q)
#pragma unroll
            for (int s = 0; s < BK / 64; ++s) R.m[q][s] = mrow[16 * q * (BK / 32) + 2 * s + (g >> 1)];
    }
    if constexpr (XT) {
        // whole X rows: instruction v of group h reads rows 16h + 4v .. +3 of the tile column (16
        // chunks of 16 bytes each, full cache lines); x_fragments moves them into the operand layout
        static_assert(BK == 128, "X rows of 128-wide tiles");
#pragma unroll
        for (int h = 0; h < MG; ++h)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = 16 * h + 4 * v + (lane >> 4);
                R.x[h][v] = ld16(a.X + (row < a.M ? row : a.M - 1) * a.ldx + (int64_t)tk * BK + 8 * (lane & 15));
            }
    } else {
#pragma unroll
        for (int u = 0; u < BK / 32; ++u) R.x[0][u] = ld16(xrow + (int64_t)tk * BK + koff<SP>(u, g));
    }
    return type;
}

// X chunks loaded as whole rows (lane L: row 4v + L/16, chunk L%16 of register v) into the operand
// layout (lane i + 16g, substep u: row i, chunk koff(u, g) / 8) through the wave's own 4 KB of LDS:
// row r at r * 256 bytes, chunk c in slot c ^ r, so the 16 rows a read instruction serves fall in
// distinct banks.  Fences before the writes (the previous tile's reads of the buffer) and between
// the writes and the reads.
template <int SP>
__device__ __forceinline__ void x_fragments(u32x4 (&x)[4], uint8_t* buf, int lane) {
    wave_lds_fence();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int row = 4 * v + (lane >> 4), ch = lane & 15;
        *reinterpret_cast<u32x4*>(buf + row * 256 + 16 * (ch ^ row)) = x[v];
    }
    wave_lds_fence();
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = koff<SP>(u, g) / 8;
        x[u] = *reinterpret_cast<const u32x4*>(buf + i * 256 + 16 * (c ^ i));
    }
}

// Index records of the NT tiles of a batch starting at tile column t (clamped to the wave's last
// tile, which exists: kb < ke): independent scalar loads, issued together.
template <int NT>
__device__ __forceinline__ void load_entries(hts_tile (&E)[NT], const GemmArgs& a, int64_t t0, int t, int ke) {
#pragma unroll
    for (int s = 0; s < NT; ++s) E[s] = a.index[t0 + (t + s < ke ? t + s : ke - 1)];
}

template <typename T, int BK, int SP, int PP, int MG>
__device__ __forceinline__ void mma_tile(const TileRegs<BK, PP, MG>& R, uint32_t type, f32x4 (&acc)[MG][PP], int lane) {
    const int g = lane >> 4;
    if (type == HTS_TILE_DENSE) {
#pragma unroll
        for (int q = 0; q < PP; ++q)
#pragma unroll
            for (int u = 0; u < BK / 32; ++u)
#pragma unroll
                for (int h = 0; h < MG; ++h) acc[h][q] = mfma_dense<T>(R.a[q][u], R.x[h][u], acc[h][q]);
    } else {
#pragma unroll
        for (int q = 0; q < PP; ++q)
#pragma unroll
            for (int s = 0; s < BK / 64; ++s) {
                const uint32_t code = R.m[q][s] >> (16 * (g & 1));
                if (SP == SPARSE_SMFMAC) {
#pragma unroll
                    for (int h = 0; h < MG; ++h)
                        acc[h][q] = mfma_sparse<T, 0>(R.a[q][s], cat8(R.x[h][2 * s], R.x[h][2 * s + 1]), code, acc[h][q]);
                } else {
                    const u32x4 v = R.a[q][s];
                    const u32x4 e0 = expand_two_groups(uint2{v[0], v[1]}, code & 0xFFu);
                    const u32x4 e1 = expand_two_groups(uint2{v[2], v[3]}, (code >> 8) & 0xFFu);
#pragma unroll
                    for (int h = 0; h < MG; ++h) {
                        acc[h][q] = mfma_dense<T>(e0, R.x[h][2 * s], acc[h][q]);
                        acc[h][q] = mfma_dense<T>(e1, R.x[h][2 * s + 1], acc[h][q]);
                    }
                }
            }
    }
}

template <typename T, int BK, bool HYB, int SP, int KS, int NT, int PP, bool XT, int MG = 1>
__global__ __launch_bounds__(64 * KS) void gemm_decode_kernel(const GemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD x (= blockIdx % 8) takes blocks of PP panels [x*q + min(x, r), ...) in order
    const uint32_t P = gridDim.x, b = blockIdx.x, x = b & 7u, q = P >> 3, r = P & 7u;
    const int64_t n0 = (int64_t)(x * q + (x < r ? x : r) + (b >> 3)) * 16 * PP;
    const int64_t tn = n0 / a.bn;
    const int r0 = (int)(n0 - tn * a.bn);
    const int Tk = (int)(a.K / BK);
    const int64_t t0 = tn * Tk;
    const int kb = Tk * wave / KS, ke = Tk * (wave + 1) / KS;

    const int i = lane & 15;
    const int64_t j = i < a.M ? i : a.M - 1;
    const uint16_t* xrow = a.X + j * a.ldx;
    // per-wave LDS: X staging (XT: 4 KB per group of 16 rows), then the wave's partial sums
    constexpr int XB = XT ? MG * 16 * 256 : 0, RB = MG * PP * 64 * 16, WB = XB > RB ? XB : RB;
    __shared__ __attribute__((aligned(16))) uint8_t wbuf[KS][WB];
    f32x4 acc[MG][PP];
#pragma unroll
    for (int h = 0; h < MG; ++h)
#pragma unroll
        for (int q2 = 0; q2 < PP; ++q2) acc[h][q2] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the index records of a batch are read one batch ahead, so their latency hides under the
    // weight loads of the batch before instead of preceding them
    hts_tile E[NT] = {};
    if (HYB && kb < ke) load_entries<NT>(E, a, t0, kb, ke);
    for (int t = kb; t < ke; t += NT) {
        TileRegs<BK, PP, MG> R[NT];
        uint32_t type[NT];
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) type[s] = load_tile<T, BK, HYB, SP, PP, XT, MG>(R[s], a, E[s], t + s, n0, r0, lane, xrow);
        if (HYB && t + NT < ke) load_entries<NT>(E, a, t0, t + NT, ke);
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) {
                if constexpr (XT)
#pragma unroll
                    for (int h = 0; h < MG; ++h) x_fragments<SP>(R[s].x[h], wbuf[wave] + h * 16 * 256, lane);
                mma_tile<T, BK, SP, PP, MG>(R[s], type[s], acc, lane);
            }
    }

    // the partial sums go to the wave's own LDS (after its last X staging reads), then the KS
    // partials of each output are added in wave order
    wave_lds_fence();
    f32x4* red = reinterpret_cast<f32x4*>(wbuf[wave]);
#pragma unroll
    for (int h = 0; h < MG; ++h)
#pragma unroll
        for (int q2 = 0; q2 < PP; ++q2) red[(h * PP + q2) * 64 + lane] = acc[h][q2];
    __syncthreads();
    for (int o = threadIdx.x; o < 256 * PP * MG; o += 64 * KS) {
        // output (row rr of panel q2, column 16h + m of Y^T): lane m + 16*(rr/4), component rr%4
        const int h = o / (256 * PP), q2 = (o >> 8) % PP, m = (o >> 4) & 15, rr = o & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < KS; ++w)
            sum += reinterpret_cast<const f32x4*>(wbuf[w])[(h * PP + q2) * 64 + m + 16 * (rr >> 2)][rr & 3];
        const int64_t row = 16 * h + m;
        if (row < a.M) {
            const int64_t n = n0 + 16 * q2 + rr;
            if (a.gate) sum = silu_times(gate_value(a.gate, row * a.ldg + n, a.y_dtype), sum);
            store_y1(a.Y, row * a.ldy + n, a.y_dtype, sum);
        }
    }
}

// X rows through LDS (x_fragments) from this M on (HTS_DECODE_XT_MIN_M overrides; 17 = never).
// With few rows the operand-layout loads touch few cache lines and the LDS round trip only adds
// latency; with many, each such load touches up to 16 half-used lines.  Measured (bf16, 128x128
// tiles), staged / direct: 7B up (11008 x 4096) M=16 21.6 / 24.6 us, M=8 19.0 / 20.6, M=6
// 18.6 / 19.4, M=4 18.4 / 18.8, M=2 18.4 / 17.7; 4096 x 4096 M=16 9.7 / 10.5, M=6 8.53 / 8.47,
// M=5 8.51 / 8.23.
int decode_xt_min_m() {
    const char* v = getenv("HTS_DECODE_XT_MIN_M");
    if (v && *v) {
        const long x = strtol(v, nullptr, 10);
        if (x >= 1 && x <= 17) return (int)x;
    }
    return 6;
}

template <typename T, int BK, bool HYB, int SP, int KS, int NT, int PP>
void launch6(const GemmArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    if constexpr (BK == 128 && NT <= 2 && KS <= 8) {
        if (a.M > 16) {             // two groups of 16 X rows per weight fragment (M <= 32)
            gemm_decode_kernel<T, BK, HYB, SP, KS, NT, PP, true, 2><<<grid, block, 0, s>>>(a);
            return;
        }
        if (a.M >= decode_xt_min_m()) {
            gemm_decode_kernel<T, BK, HYB, SP, KS, NT, PP, true><<<grid, block, 0, s>>>(a);
            return;
        }
    }
    gemm_decode_kernel<T, BK, HYB, SP, KS, NT, PP, false><<<grid, block, 0, s>>>(a);
}

template <typename T, int BK, bool HYB, int SP, int KS, int PP>
hipError_t launch5(const GemmArgs& a, int nt, hipStream_t s) {
    const dim3 grid((unsigned)(a.N / (16 * PP))), block(64 * KS);
    // nt counts 128-wide tile columns; a 64-wide tile is half as many bytes.  With 16 waves
    // (at most 128 registers per lane) only the 2-column batch fits without spills.
    if constexpr (KS < 16 && PP == 1) {
        if (nt >= 4 && a.M <= 16) {
            launch6<T, BK, HYB, SP, KS, 4 * 128 / BK, PP>(a, grid, block, s);
            return hipGetLastError();
        }
    }
    if constexpr (BK == 128) {
        if (nt == 1) {
            launch6<T, BK, HYB, SP, KS, 1, PP>(a, grid, block, s);
            return hipGetLastError();
        }
    }
    launch6<T, BK, HYB, SP, KS, 2 * 128 / BK, PP>(a, grid, block, s);
    return hipGetLastError();
}

// pp: 16-row panels per workgroup (1 or 2; 2 shares each X fragment between two panels and
// needs 32 | N, which tiles of 64 or 128 rows give)
template <typename T, int BK, bool HYB, int SP>
hipError_t launch4(const GemmArgs& a, int ksplit, int nt, int pp, hipStream_t s) {
    if (pp == 2) {
        if (ksplit >= 8) return launch5<T, BK, HYB, SP, 8, 2>(a, nt, s);
        return launch5<T, BK, HYB, SP, 4, 2>(a, nt, s);
    }
    if (ksplit >= 16 && a.M <= 16) return launch5<T, BK, HYB, SP, 16, 1>(a, nt, s);
    if (ksplit >= 8) return launch5<T, BK, HYB, SP, 8, 1>(a, nt, s);
    return launch5<T, BK, HYB, SP, 4, 1>(a, nt, s);
}

template <typename T, int BK, bool HYB>
hipError_t launch3(const GemmArgs& a, int ksplit, int nt, int pp, int sp, hipStream_t s) {
    return sp == SPARSE_SMFMAC ? launch4<T, BK, HYB, SPARSE_SMFMAC>(a, ksplit, nt, pp, s)
                               : launch4<T, BK, HYB, SPARSE_DECOMPRESS>(a, ksplit, nt, pp, s);
}

template <typename T>
hipError_t launch2(const GemmArgs& a, int ksplit, int nt, int pp, int sp, hipStream_t s) {
    const bool hyb = a.index != nullptr;
    if (a.bk == 128)
        return hyb ? launch3<T, 128, true>(a, ksplit, nt, pp, sp, s) : launch3<T, 128, false>(a, ksplit, nt, pp, sp, s);
    return hyb ? launch3<T, 64, true>(a, ksplit, nt, pp, sp, s) : launch3<T, 64, false>(a, ksplit, nt, pp, sp, s);
}

// ---------------------------------------------------------------------------------------
// 8-bit (E4M3) weights and activations, 128x128 tiles.  Same schedule as above; a tile of a
// 16-row panel is one 16x16x128 instruction.  Lane L = i + 16g (weights: row i; X: row j = i):
//   dense tile: bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the 128-byte tile row, and the
//               same bytes of the X row's 128-byte tile column
//   2:4 tile  : stored bytes [16g, 16g+16) of the 64-byte tile row (dense k in [32g, 32g+32))
//               and code word g of the row's four words -- exactly the sparse instruction's A
//               operand and index; X as for a dense tile.
template <int PP, int MG = 1>
struct TileRegs8 {
    u32x4 a[PP][2];   // per panel: dense: the two chunks; 2:4: a[q][0] = 16 stored bytes
    uint32_t m[PP];   // per panel: 2:4 code word
    u32x4 x[MG][2];   // X chunks of MG groups of 16 rows, shared by the PP panels
};

template <bool HYB, int PP, bool XT, int MG>
__device__ __forceinline__ uint32_t load_tile8(TileRegs8<PP, MG>& R, const GemmArgs& a, const hts_tile& e, int tk,
                                               int64_t n0, int r0, int lane, const uint8_t* xrow) {
    const int i = lane & 15, g = lane >> 4;
    uint32_t type = HTS_TILE_DENSE;
    uint32_t moff = 0;
    if (HYB) {
        type = e.type;
        moff = e.meta_off;
    }
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(a.values) + e.val_off;
    if (!HYB) {        // row-major W: lane i reads row i
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.W) + (n0 + i) * a.ldw + (int64_t)tk * 128;
#pragma unroll
        for (int q = 0; q < PP; ++q) {
            R.a[q][0] = ld16(base + 16 * q * a.ldw + 16 * g);
            R.a[q][1] = ld16(base + 16 * q * a.ldw + 64 + 16 * g);
        }
    } else if (type == HTS_TILE_DENSE) {
        // packed tile: 16-row panels of 128-byte rows, chunk c of panel row i at (16 c + i) * 16 bytes
        const uint8_t* panel = vb + (int64_t)r0 * 128;
#pragma unroll
        for (int q = 0; q < PP; ++q) {
            R.a[q][0] = ldw16(panel + 16 * q * 128 + (16 * g + i) * 16);
            R.a[q][1] = ldw16(panel + 16 * q * 128 + (16 * (4 + g) + i) * 16);
        }
    } else {
        const uint32_t* mrow = a.meta + moff + (int64_t)(r0 + i) * 4;
        const uint8_t* panel = vb + (int64_t)r0 * 64;   // stored rows: 64 bytes
#pragma unroll
        for (int q = 0; q < PP; ++q) R.a[q][0] = ldw16(panel + 16 * q * 64 + (16 * g + i) * 16);
#pragma unroll
        for (int q = 0; q < PP; ++q) R.m[q] = mrow[64 * q + g];
    }
    if constexpr (XT) {
        // whole X rows: instruction v of group h reads rows 16h + 8v .. +7 of the 128-byte tile column
        const uint8_t* X8 = reinterpret_cast<const uint8_t*>(a.X);
#pragma unroll
        for (int h = 0; h < MG; ++h)
#pragma unroll
            for (int v = 0; v < 2; ++v) {
                const int64_t row = 16 * h + 8 * v + (lane >> 3);
                R.x[h][v] = ld16(X8 + (row < a.M ? row : a.M - 1) * a.ldx + (int64_t)tk * 128 + 16 * (lane & 7));
            }
    } else {
        static_assert(MG == 1, "two X row groups are loaded as whole rows");
        R.x[0][0] = ld16(xrow + (int64_t)tk * 128 + 16 * g);
        R.x[0][1] = ld16(xrow + (int64_t)tk * 128 + 64 + 16 * g);
    }
    return type;
}

// 8-bit X rows (lane L: row 8v + L/8, chunk L%8 of register v) into the operand layout (lane i + 16g:
// chunks g and 4 + g of row i) through the wave's 2 KB of LDS: row r at r * 128 bytes, chunk c in
// slot c ^ ((r >> 1) & 7), so the 16 rows a read serves fall in distinct banks.
__device__ __forceinline__ void x_fragments8(u32x4 (&x)[2], uint8_t* buf, int lane) {
    wave_lds_fence();
#pragma unroll
    for (int v = 0; v < 2; ++v) {
        const int row = 8 * v + (lane >> 3), ch = lane & 7;
        *reinterpret_cast<u32x4*>(buf + row * 128 + 16 * (ch ^ ((row >> 1) & 7))) = x[v];
    }
    wave_lds_fence();
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = 4 * h + g;
        x[h] = *reinterpret_cast<const u32x4*>(buf + i * 128 + 16 * (c ^ ((i >> 1) & 7)));
    }
}

template <int PP, int MG>
__device__ __forceinline__ void mma_tile8(const TileRegs8<PP, MG>& R, uint32_t type, f32x4 (&acc)[MG][PP]) {
    if (type == HTS_TILE_DENSE) {
#pragma unroll
        for (int h = 0; h < MG; ++h)
#pragma unroll
            for (int q = 0; q < PP; ++q) {
                acc[h][q] = mfma_dense<FP8T>(R.a[q][0], R.x[h][0], acc[h][q]);
                acc[h][q] = mfma_dense<FP8T>(R.a[q][1], R.x[h][1], acc[h][q]);
            }
    } else {
#pragma unroll
        for (int h = 0; h < MG; ++h) {
            const u32x8 xb = cat8(R.x[h][0], R.x[h][1]);
#pragma unroll
            for (int q = 0; q < PP; ++q) acc[h][q] = mfma_fp8_sparse(R.a[q][0], xb, R.m[q], acc[h][q]);
        }
    }
}

template <bool HYB, int KS, int NT, int PP, bool XT, int MG = 1>
__global__ __launch_bounds__(64 * KS) void gemm_decode8_kernel(const GemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t P = gridDim.x, b = blockIdx.x, x = b & 7u, q = P >> 3, r = P & 7u;
    const int64_t n0 = (int64_t)(x * q + (x < r ? x : r) + (b >> 3)) * 16 * PP;
    const int64_t tn = n0 / a.bn;
    const int r0 = (int)(n0 - tn * a.bn);
    const int Tk = (int)(a.K / 128);
    const int64_t t0 = tn * Tk;
    const int kb = Tk * wave / KS, ke = Tk * (wave + 1) / KS;

    const int i = lane & 15;
    const int64_t j = i < a.M ? i : a.M - 1;
    const uint8_t* xrow = reinterpret_cast<const uint8_t*>(a.X) + j * a.ldx;
    // per-wave LDS: X staging (XT: 2 KB per group of 16 rows), then the wave's partial sums
    constexpr int XB = XT ? MG * 16 * 128 : 0, RB = MG * PP * 64 * 16, WB = XB > RB ? XB : RB;
    __shared__ __attribute__((aligned(16))) uint8_t wbuf[KS][WB];
    f32x4 acc[MG][PP];
#pragma unroll
    for (int h = 0; h < MG; ++h)
#pragma unroll
        for (int q2 = 0; q2 < PP; ++q2) acc[h][q2] = f32x4{0.f, 0.f, 0.f, 0.f};
    hts_tile E[NT] = {};
    if (HYB && kb < ke) load_entries<NT>(E, a, t0, kb, ke);
    for (int t = kb; t < ke; t += NT) {
        TileRegs8<PP, MG> R[NT];
        uint32_t type[NT];
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) type[s] = load_tile8<HYB, PP, XT, MG>(R[s], a, E[s], t + s, n0, r0, lane, xrow);
        if (HYB && t + NT < ke) load_entries<NT>(E, a, t0, t + NT, ke);
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) {
                if constexpr (XT)
#pragma unroll
                    for (int h = 0; h < MG; ++h) x_fragments8(R[s].x[h], wbuf[wave] + h * 16 * 128, lane);
                mma_tile8<PP, MG>(R[s], type[s], acc);
            }
    }

    // partial sums through the wave's own LDS (after its last X staging reads), added in wave order
    wave_lds_fence();
    f32x4* red = reinterpret_cast<f32x4*>(wbuf[wave]);
#pragma unroll
    for (int h = 0; h < MG; ++h)
#pragma unroll
        for (int q2 = 0; q2 < PP; ++q2) red[(h * PP + q2) * 64 + lane] = acc[h][q2];
    __syncthreads();
    for (int o = threadIdx.x; o < 256 * PP * MG; o += 64 * KS) {
        const int h = o / (256 * PP), q2 = (o >> 8) % PP, m = (o >> 4) & 15, rr = o & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < KS; ++w)
            sum += reinterpret_cast<const f32x4*>(wbuf[w])[(h * PP + q2) * 64 + m + 16 * (rr >> 2)][rr & 3];
        const int64_t row = 16 * h + m;
        if (row < a.M) {
            const int64_t n = n0 + 16 * q2 + rr;
            if (a.gate) sum = silu_times(gate_value(a.gate, row * a.ldg + n, a.y_dtype), sum);
            store_y1(a.Y, row * a.ldy + n, a.y_dtype, sum);
        }
    }
}

template <bool HYB, int KS, int NT, int PP>
void launch8x(const GemmArgs& a, dim3 grid, dim3 block, hipStream_t s) {
    if constexpr (NT <= 4 && KS <= 8) {
        if (a.M > 16) {             // two groups of 16 X rows per weight fragment (M <= 32)
            gemm_decode8_kernel<HYB, KS, NT, PP, true, 2><<<grid, block, 0, s>>>(a);
            return;
        }
    }
    if (a.M >= decode_xt_min_m()) gemm_decode8_kernel<HYB, KS, NT, PP, true><<<grid, block, 0, s>>>(a);
    else gemm_decode8_kernel<HYB, KS, NT, PP, false><<<grid, block, 0, s>>>(a);
}

template <bool HYB, int KS, int PP>
hipError_t launch8_nt(const GemmArgs& a, int nt, hipStream_t s) {
    const dim3 grid((unsigned)(a.N / (16 * PP))), block(64 * KS);
    // nt counts 16-bit 128x128 tile columns; an 8-bit tile column is half the bytes
    if constexpr (KS < 16 && PP == 1) {
        if (nt >= 4 && a.M <= 16) {
            launch8x<HYB, KS, 8, PP>(a, grid, block, s);
            return hipGetLastError();
        }
    }
    launch8x<HYB, KS, 4, PP>(a, grid, block, s);
    return hipGetLastError();
}

template <bool HYB>
hipError_t launch8(const GemmArgs& a, int ksplit, int nt, int pp, hipStream_t s) {
    if (pp == 2) {
        if (ksplit >= 8) return launch8_nt<HYB, 8, 2>(a, nt, s);
        return launch8_nt<HYB, 4, 2>(a, nt, s);
    }
    if (ksplit >= 16 && a.M <= 16) return launch8_nt<HYB, 16, 1>(a, nt, s);
    if (ksplit >= 8) return launch8_nt<HYB, 8, 1>(a, nt, s);
    return launch8_nt<HYB, 4, 1>(a, nt, s);
}

// ---------------------------------------------------------------------------------------
// 16-bit weights in 32-wide tiles (bk = 32).  A tile of a 16-row panel is one 16x16x32 MFMA:
// lane L = i + 16g takes k in [8g, 8g+8) of the tile, weights of row i and X of row j = i.
// A 2:4 tile row holds 16 stored values and one code word; lane group g expands groups 2g and
// 2g+1 (stored values 4g..4g+3, code byte g) in registers into its 8 dense weights -- the
// sparse instruction spans 64 k, two such tiles of which may differ in type.
template <int PP>
struct TileRegs32 {
    u32x4 a[PP];      // per panel: dense: 8 weights; 2:4: the 4 stored values in a[q][0..1]
    uint32_t m[PP];   // per panel: 2:4 code word of the row
    u32x4 x;          // X: 8 values of row j
};

template <bool HYB, int PP>
__device__ __forceinline__ uint32_t load_tile32(TileRegs32<PP>& R, const GemmArgs& a, const hts_tile& e, int tk,
                                                int64_t n0, int r0, int lane, const uint16_t* xrow) {
    const int i = lane & 15, g = lane >> 4;
    uint32_t type = HTS_TILE_DENSE;
    uint32_t moff = 0;
    if (HYB) {
        type = e.type;
        moff = e.meta_off;
    }
    if (!HYB) {        // row-major W: lane i reads row i
        const uint16_t* base = a.W + (n0 + i) * a.ldw + (int64_t)tk * 32;
#pragma unroll
        for (int q = 0; q < PP; ++q) R.a[q] = ld16(base + 16 * q * a.ldw + 8 * g);
    } else if (type == HTS_TILE_DENSE) {
        // packed tile: 16-row panels of 32-value rows (4 chunks), chunk c of panel row i at 16 c + i
        const uint16_t* panel = a.values + e.val_off + (int64_t)r0 * 32;
#pragma unroll
        for (int q = 0; q < PP; ++q) R.a[q] = ldw16(panel + 16 * q * 32 + (16 * g + i) * 8);
    } else {
        // stored rows of 16 values (2 chunks): the 4 values of group pair g are half g % 2 of chunk g / 2
        const uint32_t* mrow = a.meta + moff + (r0 + i);
        const uint16_t* panel = a.values + e.val_off + (int64_t)r0 * 16;
#pragma unroll
        for (int q = 0; q < PP; ++q) {
            const uint2 v = *reinterpret_cast<const uint2*>(panel + 16 * q * 16 + (16 * (g >> 1) + i) * 8 + 4 * (g & 1));
            R.a[q] = u32x4{v.x, v.y, 0u, 0u};
            R.m[q] = mrow[16 * q];
        }
    }
    R.x = ld16(xrow + (int64_t)tk * 32 + 8 * g);
    return type;
}

template <typename T, int PP>
__device__ __forceinline__ void mma_tile32(const TileRegs32<PP>& R, uint32_t type, f32x4 (&acc)[PP], int lane) {
    const int g = lane >> 4;
    if (type == HTS_TILE_DENSE) {
#pragma unroll
        for (int q = 0; q < PP; ++q) acc[q] = mfma_dense<T>(R.a[q], R.x, acc[q]);
    } else {
#pragma unroll
        for (int q = 0; q < PP; ++q)
            acc[q] = mfma_dense<T>(expand_two_groups(uint2{R.a[q][0], R.a[q][1]}, (R.m[q] >> (8 * g)) & 0xFFu),
                                   R.x, acc[q]);
    }
}

template <typename T, bool HYB, int KS, int NT, int PP>
__global__ __launch_bounds__(64 * KS) void gemm_decode32_kernel(const GemmArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t P = gridDim.x, b = blockIdx.x, x = b & 7u, q = P >> 3, r = P & 7u;
    const int64_t n0 = (int64_t)(x * q + (x < r ? x : r) + (b >> 3)) * 16 * PP;
    const int64_t tn = n0 / a.bn;
    const int r0 = (int)(n0 - tn * a.bn);
    const int Tk = (int)(a.K / 32);
    const int64_t t0 = tn * Tk;
    const int kb = Tk * wave / KS, ke = Tk * (wave + 1) / KS;

    const int i = lane & 15;
    const int64_t j = i < a.M ? i : a.M - 1;
    const uint16_t* xrow = a.X + j * a.ldx;
    f32x4 acc[PP];
#pragma unroll
    for (int q2 = 0; q2 < PP; ++q2) acc[q2] = f32x4{0.f, 0.f, 0.f, 0.f};
    hts_tile E[NT] = {};
    if (HYB && kb < ke) load_entries<NT>(E, a, t0, kb, ke);
    for (int t = kb; t < ke; t += NT) {
        TileRegs32<PP> R[NT];
        uint32_t type[NT];
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) type[s] = load_tile32<HYB, PP>(R[s], a, E[s], t + s, n0, r0, lane, xrow);
        if (HYB && t + NT < ke) load_entries<NT>(E, a, t0, t + NT, ke);
#pragma unroll
        for (int s = 0; s < NT; ++s)
            if (t + s < ke) mma_tile32<T, PP>(R[s], type[s], acc, lane);
    }

    __shared__ f32x4 red[KS][PP][64];
#pragma unroll
    for (int q2 = 0; q2 < PP; ++q2) red[wave][q2][lane] = acc[q2];
    __syncthreads();
    for (int o = threadIdx.x; o < 256 * PP; o += 64 * KS) {
        const int q2 = o >> 8, m = (o >> 4) & 15, rr = o & 15;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < KS; ++w) sum += red[w][q2][m + 16 * (rr >> 2)][rr & 3];
        if (m < a.M) {
            const int64_t n = n0 + 16 * q2 + rr;
            if (a.gate) sum = silu_times(gate_value(a.gate, (int64_t)m * a.ldg + n, a.y_dtype), sum);
            store_y1(a.Y, (int64_t)m * a.ldy + n, a.y_dtype, sum);
        }
    }
}

template <typename T, bool HYB>
hipError_t launch32(const GemmArgs& a, int ksplit, int pp, hipStream_t s) {
    // eight 32-wide tile columns per batch: the bytes of two 128-wide ones
    if (pp == 2) {
        const dim3 grid((unsigned)(a.N / 32)), block(64 * (ksplit >= 8 ? 8 : 4));
        if (ksplit >= 8) gemm_decode32_kernel<T, HYB, 8, 8, 2><<<grid, block, 0, s>>>(a);
        else gemm_decode32_kernel<T, HYB, 4, 8, 2><<<grid, block, 0, s>>>(a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(a.N / 16));
    if (ksplit >= 16) gemm_decode32_kernel<T, HYB, 16, 8, 1><<<grid, dim3(1024), 0, s>>>(a);
    else if (ksplit >= 8) gemm_decode32_kernel<T, HYB, 8, 8, 1><<<grid, dim3(512), 0, s>>>(a);
    else gemm_decode32_kernel<T, HYB, 4, 8, 1><<<grid, dim3(256), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs& a, int ksplit, int nt, int pp, int sparse_path, hipStream_t s) {
    // M = 17 .. 32 runs two groups of X rows per weight fragment: 128-wide tiles
    if (a.M < 1 || a.M > 32 || (a.M > 16 && a.bk != 128)) return hipErrorInvalidValue;
    if (a.dtype == HTS_FP8_E4M3)   // 8-bit: the sparse instruction only (no expansion fallback)
        return a.index ? launch8<true>(a, ksplit, nt, pp, s) : launch8<false>(a, ksplit, nt, pp, s);
    if (a.bk == 32) {              // 32-wide tiles: expansion in registers
        (void)nt;
        (void)sparse_path;
        if (a.dtype == HTS_BF16) return a.index ? launch32<BF16T, true>(a, ksplit, pp, s) : launch32<BF16T, false>(a, ksplit, pp, s);
        return a.index ? launch32<F16T, true>(a, ksplit, pp, s) : launch32<F16T, false>(a, ksplit, pp, s);
    }
    return a.dtype == HTS_BF16 ? launch2<BF16T>(a, ksplit, nt, pp, sparse_path, s)
                               : launch2<F16T>(a, ksplit, nt, pp, sparse_path, s);
}

}  // namespace hts
