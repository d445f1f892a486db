/*
 * hts.h -- hybrid tile-sparse (dense / 2:4) linear layers on AMD Instinct MI355X (gfx950).
 *
 * The operation (page "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs",
 * section 2, core mechanism and inference/deployment): the weight W[N,K] of a
 * linear layer is cut into bn x bk tiles; a per-tile map marks each tile dense
 * (all weights kept) or 2:4 sparse (two of every four weights kept along K,
 * six possible patterns).  Dense tiles run on the dense matrix cores and 2:4
 * tiles on the sparse matrix cores, inside one product
 *
 *         Y[M,N] = X[M,K] . mask(W)^T        (fp32 accumulation)
 *
 * so that the overall sparsity can be anything from 0 % to 50 % (section 3).
 * The same page stresses that speed needs compressed storage, not zeros; the
 * packed format below is that storage.
 *
 * Conventions for every entry point
 *   - All matrices are row-major.  W is [N,K] with leading dimension ldw,
 *     X is [M,K] (ldx), Y is [M,N] (ldy); leading dimensions are in elements.
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary CPU memory, read or written only during the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Device
 *     work is enqueued on it and the call returns without waiting; results are
 *     ready when the stream reaches that point.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     (outside HTS_DEBUG mode, below), frees nothing and keeps no pointer after
 *     a call returns.
 *   - Every argument check is made on the host before anything is enqueued: a
 *     failing call has no side effect and returns a status (details in
 *     hts_last_error()).  Buffer sizes and the validity of device pointers
 *     cannot be checked cheaply and are preconditions.
 *   - Calls are thread-safe; calls that write the same buffers race.
 *   - Debug mode, environment variable HTS_DEBUG=1 (any value but "0"): before
 *     anything is enqueued, each device buffer a call touches must lie inside
 *     one device allocation of this process with the bytes the call needs
 *     (else HTS_ERR_INVALID_ARG for memory that is not device memory,
 *     HTS_ERR_SHAPE for a short buffer), and a device tile index is checked
 *     by a small kernel: every record must equal the prefix sums hts_pack_plan
 *     writes (else HTS_ERR_MAP, naming the first bad record); the values and
 *     codes buffers must then hold the sizes that index implies.  The index
 *     check synchronises the stream (it is refused during graph capture) and
 *     keeps one 24-byte result buffer per device, allocated on first use.
 *     hts_gemm_noalloc runs none of these checks.
 */
#ifndef HTS_H
#define HTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HTS_ABI_VERSION 1u

typedef enum {
    HTS_OK = 0,
    HTS_ERR_INVALID_ARG = 1,   /* null pointer where one is required, negative size, bad enum   */
    HTS_ERR_DTYPE = 2,         /* element type not supported by this entry point                */
    HTS_ERR_SHAPE = 3,         /* N, K not multiples of the tile, leading dimension too small   */
    HTS_ERR_ALIGN = 4,         /* pointer not 16-byte aligned or leading dimension not a multiple of 8 */
    HTS_ERR_MAP = 5,           /* a tile-map entry other than 0 or 1                            */
    HTS_ERR_WORKSPACE = 6,     /* workspace smaller than hts_gemm_workspace() asks for          */
    HTS_ERR_UNSUPPORTED = 7,   /* valid request this build does not implement (tile size ...)   */
    HTS_ERR_HIP = 8            /* the HIP runtime reported an error (launch failure, no device) */
} hts_status;

/* HTS_FP8_E4M3: the 8-bit OCP E4M3 format (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, no infinities; 0x7F and 0xFF are NaN, whose products are unspecified).  It serves
 * the prune-then-quantize combination (page "SparseGPT vs Wanda: one-shot LLM pruning without
 * retraining", FAQ: pruning combines with low-precision weights): W and X both 8-bit, products
 * on the 8-bit matrix instructions with fp32 accumulation, 128x128 tiles only.  Y is written as
 * HTS_F32, HTS_F16 or HTS_BF16.  The Wanda helpers and hts_silu_mul stay 16-bit. */
typedef enum { HTS_F16 = 0, HTS_BF16 = 1, HTS_F32 = 2, HTS_FP8_E4M3 = 3 } hts_dtype;

enum { HTS_TILE_DENSE = 0, HTS_TILE_SPARSE24 = 1 };

/* Shape of a tiled weight.  dtype is HTS_F16, HTS_BF16 or HTS_FP8_E4M3 (W and X share it).
 * bn, bk in {32, 64, 128} (both 128 for HTS_FP8_E4M3); N % bn == 0 and K % bk == 0 (tiles cover W
 * exactly); N*K < 2^32.  Element sizes: 2 bytes, 1 byte for HTS_FP8_E4M3; leading dimensions
 * (in elements) must be multiples of 8, of 16 for HTS_FP8_E4M3 (16 bytes either way). */
typedef struct {
    int64_t N, K;
    int32_t bn, bk;
    int32_t dtype;
    int32_t reserved;          /* must be 0 */
} hts_desc;

/* One record per tile, tiles in row-major tile order t = tn*(K/bk) + tk.
 *   val_off  : first element of the tile in `values` (elements of the weight's type)
 *   meta_off : first 32-bit word of the tile in `meta` (sparse tiles only; for a
 *              dense tile it equals the next sparse tile's offset)
 *   type     : HTS_TILE_DENSE or HTS_TILE_SPARSE24
 *   reserved : 0 */
typedef struct {
    uint32_t val_off, meta_off, type, reserved;
} hts_tile;

typedef struct {
    uint64_t values_bytes;     /* 2 * (N*K - n_sparse*bn*bk/2) */
    uint64_t meta_bytes;       /* n_sparse * bn*bk/8            */
    uint64_t index_bytes;      /* 16 * number of tiles          */
    int64_t n_sparse;          /* number of 2:4 tiles           */
} hts_sizes;

/* Packed format (bit-exact contract of hts_pack / hts_unpack):
 *   dense tile : the bn x bk weights (raw bits of W) as rows of bk values.
 *   2:4 tile   : rows of bk/2 values: for tile row r and group g of four weights (k = 4g..4g+3
 *                from the tile start) the two kept weights, lower index first, at row position
 *                2g + {0,1} (raw bits); and the 4-bit code i0 | (i1 << 2) (i0 < i1 the kept
 *                positions in the group) at bits 4*(g%8)..+3 of meta[meta_off + r*(bk/32) + g/8].
 *   Storage order of the rows of a tile (from values[val_off]): 16-row panels, one after another;
 *   each row cut into 16-byte chunks (8 values of 16 bits, 16 of 8 bits); inside a panel the
 *   chunks column by column, the panel's 16 rows consecutive in each: chunk c of row r is at
 *   ((r / 16) * 16 * row_length + (c * 16 + r % 16) * chunk_length) values.  The four chunks of
 *   16 consecutive rows that feed one matrix-core instruction are then one contiguous kilobyte.
 *   Kept pair: the two largest scores of the group, the lower index first among
 *   equal scores.  Score = |w| as binary32, or the binary32 product |w| * c[k]
 *   when a column scale c is given (the Wanda rule: weight magnitude times the
 *   norm of the input activations of that column, page "SparseGPT vs Wanda:
 *   one-shot LLM pruning without retraining", Wanda section).
 *   Unpacked, a dropped weight reads +0.0. */

uint32_t    hts_abi_version(void);
/* Static text for a status code; never NULL. */
const char* hts_status_string(int status);
/* Detail of the last failing call on this thread ("" if none).  Valid until the
 * next call on the same thread. */
const char* hts_last_error(void);

/* Host only, synchronous.  Validates the descriptor and the map (uint8, one
 * entry per tile, row-major tile order, 0 = dense, 1 = 2:4) and fills the tile
 * index (index_host may be NULL to query sizes only) and the buffer sizes.
 * Tile map: PATCH page, section 2 (per-tile dense / 2:4 decision). */
hts_status hts_pack_plan(const hts_desc* d, const uint8_t* tile_map_host,
                         hts_tile* index_host, hts_sizes* sizes);

/* Device, asynchronous.  Writes the packed values and metadata of W under the
 * index made by hts_pack_plan (copied to the device by the caller).
 * col_scale: device float[K] column scale, or NULL for magnitude scores; must be
 * finite and >= 0.  W must be finite.  meta may be NULL when n_sparse == 0.
 * Buffers: values >= sizes.values_bytes, meta >= sizes.meta_bytes. */
hts_status hts_pack(const hts_desc* d, const hts_tile* index, const void* W, int64_t ldw,
                    const float* col_scale, void* values, uint32_t* meta, void* stream);

/* Device, asynchronous.  hts_pack with the 2:4 selection given as an element mask instead
 * of selected by score: the PATCH-Tile variant keeps 2:4 patterns frozen from a one-shot
 * pruning method and learns only the tile choices (page "PATCH: Learnable Tile-level Hybrid
 * Sparsity for LLMs", section 2, variants).
 *   mask : device uint8 [N, ldm] row-major, nonzero = keep; read only inside 2:4 tiles, where
 *          each group of four (along K, aligned at the tile start) should mark exactly two
 *          weights.  16-byte aligned, ldm >= K and a multiple of 16.
 *   malformed_groups : device uint32 or NULL.  Set to the number of groups in 2:4 tiles that
 *          do not mark exactly two weights (written when the stream reaches the call).  Such a
 *          group keeps the two weights the rank rule picks with the mask as score: marked
 *          before unmarked, the lower index first among equals.
 * Other arguments, buffers and the packed format as for hts_pack. */
hts_status hts_pack_masked(const hts_desc* d, const hts_tile* index, const void* W, int64_t ldw,
                           const uint8_t* mask, int64_t ldm, void* values, uint32_t* meta,
                           uint32_t* malformed_groups, void* stream);

/* Device, asynchronous.  Inverse of hts_pack: writes mask(W) into W_out[N,K]
 * (ldw), +0.0 at the dropped positions of 2:4 tiles -- the masked weight the hybrid layer
 * computes with (page "PATCH: Learnable Tile-level Hybrid Sparsity for LLMs", section 2, core
 * mechanism: dense tiles keep every weight, 2:4 tiles zero two of every four along K).
 * values / meta: as written by hts_pack under `index`; W_out: device, 16-byte aligned, ldw >= K
 * and a multiple of 8 (16 for HTS_FP8_E4M3).  Errors as hts_pack's. */
hts_status hts_unpack(const hts_desc* d, const hts_tile* index, const void* values,
                      const uint32_t* meta, void* W_out, int64_t ldw, void* stream);

/* Host only.  Bytes of device workspace for the fastest hts_gemm path at this shape and M
 * (0 in the streaming range: M <= 32 on 128-wide tiles, else M <= 16; the
 * environment variable HTS_DECODE_MAX_M lowers it).  Two uses, in this order within the workspace:
 *  - tiles of 32 rows or 32 columns above the streaming range: the product unpacks the weight into the
 *    workspace (N*K elements, row-major, 256-byte rounded) and runs the same-library dense
 *    product on it -- the tiled kernel works on 64-row weight groups and 64-wide slices.
 *    Execution tiles below 128x128 are the tile-size ablation of the PATCH page (sections 2
 *    and 4): finer maps, less matrix-core efficiency.  This part is required.
 *  - split products: when the tiled kernel would have at most 256 output blocks (for 128x128
 *    tiles, ceil(N/128) * ceil(M/128) <= 256), the K range of every tile row is split over up
 *    to 8 workgroups that write fp32 partial products (nsplit * M * N floats, 256-byte rounded),
 *    summed in a fixed order by a second kernel.  This part is optional: with less workspace the
 *    product runs unsplit, with the same result up to fp32 rounding order. */
hts_status hts_gemm_workspace(const hts_desc* d, int64_t M, size_t* bytes);

/* Device, asynchronous.  The hybrid linear layer (page "PATCH: Learnable Tile-level Hybrid Sparsity
 * for LLMs", section 2, core mechanism and inference/deployment: per-tile dense or 2:4 weights,
 * dense tiles on the dense matrix cores and 2:4 tiles on the sparse ones, from compressed storage):
 * Y[M,N] = X[M,K] . mask(W)^T from the packed weight, fp32 accumulation, Y written as y_dtype (HTS_F32, HTS_F16 or HTS_BF16; 16-bit
 * outputs rounded to nearest even).  In the streaming range (see hts_gemm_workspace) one
 * kernel streams the weight from HBM once; above it a tiled kernel stages weight and X
 * slices through LDS.  Dense tiles use dense MFMA, 2:4 tiles
 * sparse MFMA (or in-register expansion to dense MFMA when the environment
 * variable HTS_SPARSE_PATH=decompress), both into one accumulator per output
 * tile.  M == 0 is a no-op.  ldx, ldy: multiples of 8 and 4 with ldx >= K and
 * ldy >= N.  workspace: up to the hts_gemm_workspace() bytes, 16-byte aligned, or NULL.
 * HTS_ERR_WORKSPACE only when the unpacked weight of 32-wide tiles does not fit; a workspace
 * too small for the split-product parts runs the product unsplit.  Results are deterministic
 * for a given call shape and workspace.  Calls that share a workspace must not overlap. */
hts_status hts_gemm(const hts_desc* d, const hts_tile* index, const void* values,
                    const uint32_t* meta, int64_t M, const void* X, int64_t ldx,
                    void* Y, int64_t ldy, int32_t y_dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Device, asynchronous.  The same-library dense product Y = X . W^T on a
 * row-major W[N,K] (ldw) with the same kernels and no tile index: the
 * reference point for speedups (the dense model the PATCH page measures its speed-up against,
 * section 4, results).  X, W, Y: device, 16-byte aligned; ldx, ldw >= K and ldy >= N, leading
 * dimensions multiples of 8 (16 for HTS_FP8_E4M3) and 4; y_dtype HTS_F32, HTS_F16 or HTS_BF16.
 * M == 0 is a no-op; errors as hts_gemm's.  N and K multiples of 64.  workspace: optional, as the
 * split-product part of hts_gemm's (size from hts_dense_gemm_workspace). */
hts_status hts_dense_gemm(int32_t dtype, int64_t M, int64_t N, int64_t K,
                          const void* X, int64_t ldx, const void* W, int64_t ldw,
                          void* Y, int64_t ldy, int32_t y_dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Host only.  Bytes of the optional workspace of hts_dense_gemm at this shape (0 unless the
 * product would be split, see hts_gemm_workspace). */
hts_status hts_dense_gemm_workspace(int32_t dtype, int64_t M, int64_t N, int64_t K, size_t* bytes);

/* Device, asynchronous.  hts_gemm without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  This call allocates nothing: the workspace hts_gemm would take (the fp32 parts of a
 * split product, the unpacked weight of 32-wide tiles) is a library-owned static device array of
 * 64 MiB per GPU, held from the first use on that GPU until the process ends.  The result equals
 * hts_gemm's with a workspace of hts_gemm_workspace() bytes, bit for bit.  A shape and M whose
 * hts_gemm_workspace() exceeds 64 MiB are rejected with HTS_ERR_WORKSPACE.  Every call on one GPU
 * uses the same array: calls that overlap on one GPU (different streams, threads or graphs
 * running concurrently) race and must be serialized by the caller.  Other arguments and errors as
 * hts_gemm's; HTS_ERR_HIP if the array's device address cannot be obtained. */
hts_status hts_gemm_noalloc(const hts_desc* d, const hts_tile* index, const void* values,
                            const uint32_t* meta, int64_t M, const void* X, int64_t ldx,
                            void* Y, int64_t ldy, int32_t y_dtype, void* stream);

/* Device, asynchronous.  The hybrid product with the gated-MLP step in its output stage:
 * Y[M,N] = silu(G) * (X[M,K] . mask(W)^T), silu(x) = x / (1 + e^-x), with G[M,N] (ldg) in
 * y_dtype.  The up projection of a decoder block whose linear layers are hybrid tile-sparse
 * writes silu(gate) * up in one pass instead of writing up and running hts_silu_mul (the pages
 * prune the linear layers of LLaMA models; this step is the architecture's, not the method's).
 * The product is hts_gemm's (same kernels, tiles, workspace and determinism); the output stage
 * multiplies the fp32 sum by silu(g) in fp32 and rounds once to y_dtype.  G: 16-byte aligned,
 * ldg >= N and a multiple of 4; G may be Y (each element is read, then written, by one
 * thread).  Errors as hts_gemm's, and HTS_ERR_INVALID_ARG when G is NULL with M > 0. */
hts_status hts_gemm_silu_mul(const hts_desc* d, const hts_tile* index, const void* values,
                             const uint32_t* meta, int64_t M, const void* X, int64_t ldx,
                             const void* G, int64_t ldg, void* Y, int64_t ldy, int32_t y_dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Device, asynchronous.  H[M,N] = silu(G) * U elementwise, silu(x) = x / (1 + e^-x), fp32
 * arithmetic, one round-to-nearest-even to dtype (HTS_F16 / HTS_BF16, shared by G, U and H):
 * the gated-MLP step between the gate / up projections and the down projection of a decoder
 * block whose linear layers are hybrid tile-sparse (the pages prune the linear layers of LLaMA
 * models; this step is the architecture's, not the method's).  N % 8 == 0; G, U, H 16-byte
 * aligned with leading dimensions (elements) >= N and multiples of 8.  M == 0 is a no-op. */
hts_status hts_silu_mul(int32_t dtype, int64_t M, int64_t N, const void* G, int64_t ldg, const void* U,
                        int64_t ldu, void* H, int64_t ldh, void* stream);

/* Device, asynchronous.  Wanda column scale c[k] = ||X[:,k]||_2 of calibration
 * activations X[rows,K] (ldx): squares summed in fp64 over rows in order, one
 * rounding of the square root to fp32 (Wanda section of the SparseGPT-vs-Wanda
 * page: the input activation of each weight's column). */
hts_status hts_col_norms(int32_t dtype, int64_t rows, int64_t K, const void* X, int64_t ldx,
                         float* col_scale, void* stream);

/* Device, asynchronous.  Per-tile Wanda cost: the fp64 sum of the scores a 2:4
 * mask of the tile would drop (per row, pairs summed lower index first and
 * accumulated over groups in order; rows accumulated in order).  cost: device
 * double[T]. */
hts_status hts_wanda_tile_cost(const hts_desc* d, const void* W, int64_t ldw,
                               const float* col_scale, double* cost, void* stream);

/* Device, asynchronous.  Tile map with the n_sparse lowest-cost tiles marked
 * 2:4 (ties to the lower tile number), the rest dense: the layer-wise Wanda
 * allocation of a target sparsity.  map: device uint8[T]. */
hts_status hts_wanda_map(int64_t T, const double* cost, int64_t n_sparse, uint8_t* map,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HTS_H */
