// C ABI of the hybrid tile-sparse library: argument checks, the tile index
// (prefix sums over the tile map), variant choice and kernel launches.
// Every check happens before anything is enqueued; a failing call has no effect.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include <atomic>
#include <mutex>

#include "hts.h"
#include "hts_internal.h"

namespace {

thread_local char g_err[512];

hts_status fail(hts_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

hts_status ok() {
    g_err[0] = '\0';
    return HTS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is16bit(int32_t dt) { return dt == HTS_F16 || dt == HTS_BF16; }
bool is_in(int32_t dt) { return is16bit(dt) || dt == HTS_FP8_E4M3; }
int elem_bytes(int32_t dt) { return dt == HTS_FP8_E4M3 ? 1 : 2; }
int ld_mult(int32_t dt) { return 16 / elem_bytes(dt); }   // leading dimensions: whole 16-byte chunks
bool is_out(int32_t dt) { return dt == HTS_F16 || dt == HTS_BF16 || dt == HTS_F32; }

hts_status check_desc(const hts_desc* d) {
    if (!d) return fail(HTS_ERR_INVALID_ARG, "descriptor is NULL");
    if (!is_in(d->dtype)) return fail(HTS_ERR_DTYPE, "dtype %d is not HTS_F16, HTS_BF16 or HTS_FP8_E4M3", d->dtype);
    if (d->reserved != 0) return fail(HTS_ERR_INVALID_ARG, "descriptor reserved field must be 0");
    if (d->N <= 0 || d->K <= 0) return fail(HTS_ERR_SHAPE, "N=%lld K=%lld must be positive", (long long)d->N,
                                            (long long)d->K);
    if (!((d->bn == 32 || d->bn == 64 || d->bn == 128) && (d->bk == 32 || d->bk == 64 || d->bk == 128)))
        return fail(HTS_ERR_UNSUPPORTED, "tile %dx%d: bn and bk must each be 32, 64 or 128", d->bn, d->bk);
    if (d->dtype == HTS_FP8_E4M3 && (d->bn != 128 || d->bk != 128))
        return fail(HTS_ERR_UNSUPPORTED, "tile %dx%d: 8-bit weights use 128x128 tiles", d->bn, d->bk);
    if (d->N % d->bn || d->K % d->bk)
        return fail(HTS_ERR_SHAPE, "N=%lld K=%lld are not multiples of the %dx%d tile", (long long)d->N,
                    (long long)d->K, d->bn, d->bk);
    if ((double)d->N * (double)d->K >= 4294967296.0)
        return fail(HTS_ERR_SHAPE, "N*K must be below 2^32 (32-bit value offsets)");
    return HTS_OK;
}

hts_status check_ld(int64_t ld, int64_t minv, int mult, const char* name) {
    if (ld < minv) return fail(HTS_ERR_SHAPE, "%s=%lld is smaller than %lld", name, (long long)ld, (long long)minv);
    if (ld % mult) return fail(HTS_ERR_ALIGN, "%s=%lld is not a multiple of %d", name, (long long)ld, mult);
    return HTS_OK;
}

hts_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(HTS_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(HTS_ERR_ALIGN, "%s is not 16-byte aligned", name);
    return HTS_OK;
}

hts_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(HTS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// HTS_DEBUG=1 (any value but "0"): before anything is enqueued, every device buffer a call will
// touch is checked to lie inside one allocation of this process (hipMemGetAddressRange) with the
// bytes the call needs, and a device tile index is checked by a small kernel (its records must be
// the prefix sums of hts_pack_plan: record t = record t-1 plus that tile's stored size), which
// also yields the sizes of the values and codes the index implies.  The checks synchronise the
// stream, so they are refused during graph capture.  hts_gemm_noalloc runs none of them.
bool debug_mode() {
    const char* v = getenv("HTS_DEBUG");
    return v && *v && strcmp(v, "0") != 0;
}

// Bytes of a row-major block of `rows` rows of `cols` elements of `es` bytes, leading dimension ld.
uint64_t block_bytes(int64_t rows, int64_t cols, int64_t ld, int es) {
    return rows > 0 ? (uint64_t)((rows - 1) * ld + cols) * (uint64_t)es : 0;
}

hts_status debug_range(const void* p, uint64_t bytes, const char* name) {
    if (!p || bytes == 0) return HTS_OK;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    const hipError_t e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
    if (e != hipSuccess || !base) {
        (void)hipGetLastError();   // leave no stale error for the next launch check
        return fail(HTS_ERR_INVALID_ARG, "HTS_DEBUG: %s is not device memory of this process", name);
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < lo || q - lo + bytes > size)
        return fail(HTS_ERR_SHAPE, "HTS_DEBUG: %s needs %llu bytes; its allocation ends %llu bytes after it", name,
                    (unsigned long long)bytes, (unsigned long long)(q >= lo && q - lo <= size ? size - (q - lo) : 0));
    return HTS_OK;
}

// Per-device result buffer of the index check (allocated on first use in debug mode).
class DebugIndex {
  public:
    static constexpr int kMaxDevices = 64;
    hts_status run(const hts_desc* d, const hts_tile* index, hipStream_t s, uint64_t* values_bytes,
                   uint64_t* meta_bytes) {
        const int64_t T = (d->N / d->bn) * (d->K / d->bk);
        hts_status st = debug_range(index, 16 * (uint64_t)T, "index");
        if (st) return st;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
            return fail(HTS_ERR_INVALID_ARG, "HTS_DEBUG checks synchronise the stream and cannot run during graph capture");
        std::lock_guard<std::mutex> lock(mu_);
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) return fail(HTS_ERR_HIP, "HTS_DEBUG: no current device");
        if (!buf_[dev] && (e = hipMalloc(reinterpret_cast<void**>(&buf_[dev]), sizeof(hts::IndexCheck))) != hipSuccess)
            return hip_status(e, "HTS_DEBUG: index check buffer");
        const hts::IndexCheck init = {0u, 0xFFFFFFFFu, 0u, 0u};
        hts::IndexCheck r{};
        if ((e = hipMemcpyAsync(buf_[dev], &init, sizeof init, hipMemcpyHostToDevice, s)) != hipSuccess ||
            (e = hts::launch_index_check(*d, index, buf_[dev], s)) != hipSuccess ||
            (e = hipMemcpyAsync(&r, buf_[dev], sizeof r, hipMemcpyDeviceToHost, s)) != hipSuccess ||
            (e = hipStreamSynchronize(s)) != hipSuccess)
            return hip_status(e, "HTS_DEBUG: index check");
        if (r.bad)
            return fail(HTS_ERR_MAP, "HTS_DEBUG: %u tile index records are inconsistent with the plan (first: record %u)",
                        r.bad, r.first_bad);
        *values_bytes = r.values_end * (uint64_t)elem_bytes(d->dtype);
        *meta_bytes = 4 * r.meta_end;
        return HTS_OK;
    }

  private:
    std::mutex mu_;
    hts::IndexCheck* buf_[kMaxDevices] = {};
};
DebugIndex g_debug_index;

// The packed weight's buffers: the index, then the values and codes it implies.
hts_status debug_packed(const hts_desc* d, const hts_tile* index, const void* values, const uint32_t* meta,
                        hipStream_t s, bool writes) {
    uint64_t vb = 0, mb = 0;
    hts_status st = g_debug_index.run(d, index, s, &vb, &mb);
    if (st) return st;
    if ((st = debug_range(values, vb, writes ? "values (output)" : "values"))) return st;
    if (mb && !meta) return fail(HTS_ERR_INVALID_ARG, "HTS_DEBUG: the index has 2:4 tiles but meta is NULL");
    return debug_range(meta, mb, writes ? "meta (output)" : "meta");
}


// Sparse-tile path: SMFMAC unless HTS_SPARSE_PATH=decompress.
int sparse_path() {
    const char* v = getenv("HTS_SPARSE_PATH");
    if (v && strcmp(v, "decompress") == 0) return hts::SPARSE_DECOMPRESS;
    return hts::SPARSE_SMFMAC;
}

// Largest M served by the streaming kernel: 32 on 128-wide tiles (two groups of 16 X rows per
// weight fragment), else 16.  HTS_DECODE_MAX_M (0..32) lowers it.
int64_t streaming_max_m(int32_t dtype, int bk) {
    (void)dtype;
    const int64_t lim = bk == 128 ? 32 : 16;
    const char* v = getenv("HTS_DECODE_MAX_M");
    if (v && *v) {
        long x = strtol(v, nullptr, 10);
        if (x >= 0 && x <= 32) return x < lim ? x : lim;
    }
    return lim;
}

// Tiles of 32 rows or 32 columns are below the tiled kernel's 64-row weight groups and 64-wide
// slices: at M above the streaming range the product unpacks the weight into the workspace and
// runs the dense product on it.
bool small_tiles(const hts_desc* d) { return d->bn < 64 || d->bk < 64; }
uint64_t unpack_workspace_bytes(const hts_desc* d, int64_t M) {
    if (!small_tiles(d) || M <= streaming_max_m(d->dtype, d->bk)) return 0;
    return ((uint64_t)d->N * d->K * elem_bytes(d->dtype) + 255) & ~uint64_t(255);
}

// Launch shape of the streaming kernel.  Defaults measured on MI355X (bf16, 128x128 tiles):
//   panels per workgroup pp: 2 (each X fragment feeds two 16-row panels) when K >= 4608 and that
//     still leaves at least 160 workgroups -- K = 5120: M=16 36.9 -> 29.4 us (13824 rows), 20.1 ->
//     16.4 us (5120 rows, 160 workgroups) -- else 1 (K = 4096, 11008 rows: 17.2 us at pp = 1
//     against 20.2 at pp = 2; K = 11008, 4096 rows: 13.0 against 17.6 us at M = 1, where two
//     panels would leave 128 workgroups for 256 CUs);
//   waves per workgroup: 4 when pp = 2 still leaves >= 400 workgroups, else 8 (8-bit packed
//     weights: 4 -- 7B up, M=1: 10.3 us against 12.3 at 8);
//   tile columns per batch of loads: 1 with two panels (13B layers, M = 1 .. 16: 3-5% faster than
//     2), on rows of K >= 4608 (K = 11008, 4096 rows: M = 1 12.8 against 13.8 us), or at M > 16,
//     where two groups of X rows double the X registers and a batch of two would leave one wave
//     per SIMD; else 2.
// HTS_DECODE_PP=1|2, HTS_DECODE_KSPLIT=4|8|16 and HTS_DECODE_NT=1|2|4 override.
int decode_pp(const hts::GemmArgs& a) {
    if (a.N % 32) return 1;                  // every accepted shape has 32 | N; kept as a guard
    const char* v = getenv("HTS_DECODE_PP");
    if (v && !strcmp(v, "2")) return 2;
    if (v && !strcmp(v, "1")) return 1;
    return (a.K >= 4608 && a.N / 32 >= 160) ? 2 : 1;
}

int decode_ksplit(const hts::GemmArgs& a) {
    const char* v = getenv("HTS_DECODE_KSPLIT");
    if (v && (!strcmp(v, "4") || !strcmp(v, "8") || !strcmp(v, "16"))) return atoi(v);
    // 8-bit tiles are half the bytes: fewer, longer waves stream better -- for the packed weight
    // at every M (7B up: M=8 12.2 -> 10.8 us, M=16 12.6 -> 11.7), for a row-major one below M = 8
    // -- as long as at least 400 workgroups remain (K = 11008, 4096 rows, 256 workgroups: M = 1
    // 14.3 us with 4 waves against 9.9 with 8)
    const int wgs = (int)(a.N / (16 * decode_pp(a)));
    if (a.dtype == HTS_FP8_E4M3 && (a.index || a.M < 8) && wgs >= 400) return 4;
    return (decode_pp(a) == 2 && wgs >= 400) ? 4 : 8;
}

int decode_nt(const hts::GemmArgs& a) {
    const char* v = getenv("HTS_DECODE_NT");
    if (v && (!strcmp(v, "1") || !strcmp(v, "2") || !strcmp(v, "4"))) return atoi(v);
    return (a.M > 16 || decode_pp(a) == 2 || a.K >= 4608) ? 1 : 2;
}



// Split products (tiled kernel, default block shape).  A workgroup alone on its CU takes about as
// long per 64-wide slice as each of two sharing one, so a grid of at most 256 blocks (one per CU)
// leaves half the chip's slots empty and its run time is set by the slices per block.  Then the
// slices of each tile row are split over nsplit workgroups -- at most 512 in all (two per CU), at
// least 4 slices and at most 8 parts -- and a second kernel sums their fp32 parts in a fixed
// order.  Measured on the 7B up-projection (11008 x 4096, bf16, 86 tile rows), split / unsplit:
// M = 17 23.7 / 60.5 us (5 parts), 64 28.4 / 60.6, 128 37.2 / 61.3, 256 54.4 / 62.1 (2 parts);
// at 258 and more blocks (M > 256 here) splitting was slower at every count tried.
// HTS_PREFILL_SPLIT=1..16 overrides.  block_rows: weight rows per block of the launch.
int prefill_split(int64_t M, int64_t N, int64_t K, int32_t dtype, int bk, int block_rows) {
    if (M <= streaming_max_m(dtype, bk)) return 1;
    const int64_t slices = K * elem_bytes(dtype) / 128;
    const char* v = getenv("HTS_PREFILL_SPLIT");
    if (v && *v) {
        const long x = strtol(v, nullptr, 10);
        if (x >= 1 && x <= 16) return (int)(x < slices ? x : slices);
    }
    const int bm = hts::prefill_block_m(M, N, dtype, block_rows);
    const int64_t blocks = ((N + block_rows - 1) / block_rows) * ((M + bm - 1) / bm);
    if (blocks > 256) return 1;
    int64_t sp = 512 / blocks;
    if (sp > 8) sp = 8;
    while (sp > 1 && slices / sp < 4) --sp;
    return (int)sp;
}

uint64_t split_bytes(int64_t M, int64_t N, int nsplit) {
    if (nsplit <= 1) return 0;
    return ((uint64_t)nsplit * M * N * 4 + 255) & ~uint64_t(255);
}

// Attach the partial-product buffer when the workspace holds it; otherwise run unsplit.
void attach_split(hts::GemmArgs& a, int nsplit, void* ws, size_t ws_bytes) {
    a.nsplit = 1;
    a.part = nullptr;
    if (nsplit > 1 && ws && ws_bytes >= split_bytes(a.M, a.N, nsplit)) {
        a.nsplit = nsplit;
        a.part = static_cast<float*>(ws);
    }
}

hts_status run_gemm(const hts::GemmArgs& a, hipStream_t s) {
    hipError_t e;
    if (a.M <= streaming_max_m(a.dtype, a.bk)) {
        e = hts::launch_gemm_decode(a, decode_ksplit(a), decode_nt(a), decode_pp(a), sparse_path(), s);
    } else {
        // the tiled kernel addresses X rows (and rows of a row-major W) by 32-bit byte offsets
        // from its block's first row
        if (a.ldx > (int64_t(1) << 24) || (!a.index && a.ldw > (int64_t(1) << 24)))
            return fail(HTS_ERR_UNSUPPORTED, "leading dimension above 2^24 elements at M > %lld",
                        (long long)streaming_max_m(a.dtype, a.bk));
        if (a.index && a.K / a.bk > hts::kMaxTileColsPerRow)
            return fail(HTS_ERR_UNSUPPORTED, "K/bk=%lld tile columns exceed the %d of one tile row the tiled kernel holds",
                        (long long)(a.K / a.bk), hts::kMaxTileColsPerRow);
        e = hts::launch_gemm_prefill(a, sparse_path(), s);
    }
    return hip_status(e, "product kernel launch");
}

// hts_gemm and hts_gemm_silu_mul (gate: G[M,N] in y_dtype, or nullptr)
hts_status gemm_impl(const hts_desc* d, const hts_tile* index, const void* values, const uint32_t* meta, int64_t M,
                     const void* X, int64_t ldx, const void* gate, int64_t ldg, void* Y, int64_t ldy, int32_t y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream, bool debug_ok = true) {
    hts_status st = check_desc(d);
    if (st) return st;
    if (M < 0) return fail(HTS_ERR_SHAPE, "M=%lld is negative", (long long)M);
    if (!is_out(y_dtype)) return fail(HTS_ERR_DTYPE, "y_dtype %d is not F32, F16 or BF16", y_dtype);
    if ((st = check_ptr(index, "index")) || (st = check_ptr(values, "values"))) return st;
    if (meta && !aligned16(meta)) return fail(HTS_ERR_ALIGN, "meta is not 16-byte aligned");
    if ((st = check_ld(ldx, d->K, ld_mult(d->dtype), "ldx")) || (st = check_ld(ldy, d->N, 4, "ldy"))) return st;
    if (M == 0) return ok();
    if ((st = check_ptr(X, "X")) || (st = check_ptr(Y, "Y"))) return st;
    if (gate && (st = check_ptr(gate, "G"))) return st;
    if (debug_ok && debug_mode()) {
        const int ys = y_dtype == HTS_F32 ? 4 : 2;
        if ((st = debug_packed(d, index, values, meta, static_cast<hipStream_t>(stream), false)) ||
            (st = debug_range(X, block_bytes(M, d->K, ldx, elem_bytes(d->dtype)), "X")) ||
            (st = debug_range(Y, block_bytes(M, d->N, ldy, ys), "Y")) ||
            (st = debug_range(gate, block_bytes(M, d->N, ldg, ys), "G")) ||
            (st = debug_range(workspace, workspace_bytes, "workspace")))
            return st;
    }
    const uint64_t ws = unpack_workspace_bytes(d, M);
    if (ws) {
        if (!workspace || workspace_bytes < ws)
            return fail(HTS_ERR_WORKSPACE, "tiles of %dx%d at M=%lld need a %llu-byte workspace (got %zu)", d->bn,
                        d->bk, (long long)M, (unsigned long long)ws, workspace_bytes);
        if (!aligned16(workspace)) return fail(HTS_ERR_ALIGN, "workspace is not 16-byte aligned");
        if (d->N % 64 || d->K % 64)
            return fail(HTS_ERR_UNSUPPORTED, "the unpacked product needs N and K multiples of 64");
        // the unpacked weight, row-major with ldw = K, then the same-library dense product on it
        hipError_t e = hts::launch_unpack(*d, index, static_cast<const uint16_t*>(values), meta,
                                          static_cast<uint16_t*>(workspace), d->K, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return hip_status(e, "unpack kernel launch");
        hts::GemmArgs a{};
        a.dtype = d->dtype;
        a.y_dtype = y_dtype;
        a.M = M;
        a.N = d->N;
        a.K = d->K;
        a.bn = 64;
        a.bk = (d->K % 128 == 0) ? 128 : 64;
        a.W = static_cast<const uint16_t*>(workspace);
        a.ldw = d->K;
        a.X = static_cast<const uint16_t*>(X);
        a.ldx = ldx;
        a.Y = Y;
        a.ldy = ldy;
        a.gate = gate;
        a.ldg = ldg;
        attach_split(a, prefill_split(M, d->N, d->K, d->dtype, a.bk, 128), static_cast<uint8_t*>(workspace) + ws,
                     workspace_bytes - ws);
        return run_gemm(a, static_cast<hipStream_t>(stream));
    }
    if (workspace && !aligned16(workspace)) return fail(HTS_ERR_ALIGN, "workspace is not 16-byte aligned");
    hts::GemmArgs a{};
    a.dtype = d->dtype;
    a.y_dtype = y_dtype;
    a.M = M;
    a.N = d->N;
    a.K = d->K;
    a.bn = d->bn;
    a.bk = d->bk;
    a.index = index;
    a.values = static_cast<const uint16_t*>(values);
    a.meta = meta;
    a.X = static_cast<const uint16_t*>(X);
    a.ldx = ldx;
    a.Y = Y;
    a.ldy = ldy;
    a.gate = gate;
    a.ldg = ldg;
    attach_split(a,
                 prefill_split(M, d->N, d->K, d->dtype, d->bk,
                               d->dtype == HTS_FP8_E4M3 ? 128 : hts::prefill_weight_rows(d->bn)),
                 workspace, workspace_bytes);
    return run_gemm(a, static_cast<hipStream_t>(stream));
}

// Scratch of hts_gemm_noalloc: library-owned device memory, one copy per GPU (each device holds
// its own instance of a __device__ array, at its own address, from module load until the process
// ends).  Host code never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

class ScratchAddress {
  public:
    static constexpr int kMaxDevices = 64;
    hts_status get(void** out) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return fail(HTS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        if (dev < 0 || dev >= kMaxDevices) return fail(HTS_ERR_HIP, "device %d beyond the %d supported", dev, kMaxDevices);
        void* p = ptr_[dev].load(std::memory_order_acquire);
        if (!p) {
            std::lock_guard<std::mutex> lock(mu_);
            p = ptr_[dev].load(std::memory_order_relaxed);
            if (!p) {
                e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
                if (e != hipSuccess || !p)
                    return fail(HTS_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
                ptr_[dev].store(p, std::memory_order_release);
            }
        }
        *out = p;
        return HTS_OK;
    }

  private:
    std::mutex mu_;
    std::atomic<void*> ptr_[kMaxDevices] = {};
};
ScratchAddress g_scratch;

// Workspace bytes hts_gemm uses at this shape and M (what hts_gemm_workspace reports).
uint64_t gemm_workspace_bytes(const hts_desc* d, int64_t M) {
    const uint64_t ws = unpack_workspace_bytes(d, M);
    // the unpacked weight (tiles of 32), then the parts of a split product
    const int br = (ws || d->dtype == HTS_FP8_E4M3) ? 128 : hts::prefill_weight_rows(d->bn);
    const int bk = ws ? ((d->K % 128 == 0) ? 128 : 64) : d->bk;   // the unpacked product's slices
    return ws + split_bytes(M, d->N, prefill_split(M, d->N, d->K, d->dtype, bk, br));
}

}  // namespace

extern "C" {

uint32_t hts_abi_version(void) { return HTS_ABI_VERSION; }

const char* hts_status_string(int s) {
    switch (s) {
        case HTS_OK: return "ok";
        case HTS_ERR_INVALID_ARG: return "invalid argument";
        case HTS_ERR_DTYPE: return "unsupported element type";
        case HTS_ERR_SHAPE: return "invalid shape";
        case HTS_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case HTS_ERR_MAP: return "invalid tile map entry";
        case HTS_ERR_WORKSPACE: return "workspace too small";
        case HTS_ERR_UNSUPPORTED: return "unsupported configuration";
        case HTS_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* hts_last_error(void) { return g_err; }

hts_status hts_pack_plan(const hts_desc* d, const uint8_t* tile_map_host, hts_tile* index_host, hts_sizes* sizes) {
    hts_status st = check_desc(d);
    if (st) return st;
    if (!tile_map_host) return fail(HTS_ERR_INVALID_ARG, "tile map is NULL");
    if (!sizes) return fail(HTS_ERR_INVALID_ARG, "sizes is NULL");
    const int64_t T = (d->N / d->bn) * (d->K / d->bk);
    for (int64_t t = 0; t < T; ++t)
        if (tile_map_host[t] > 1)
            return fail(HTS_ERR_MAP, "tile map entry %lld is %u (must be 0 or 1)", (long long)t, tile_map_host[t]);
    const uint64_t dense = (uint64_t)d->bn * d->bk, sparse = dense / 2, mwords = dense / 32;
    uint64_t voff = 0, moff = 0;
    int64_t ns = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (index_host) {
            index_host[t].val_off = (uint32_t)voff;
            index_host[t].meta_off = (uint32_t)moff;
            index_host[t].type = tile_map_host[t];
            index_host[t].reserved = 0;
        }
        if (tile_map_host[t] == HTS_TILE_SPARSE24) {
            voff += sparse;
            moff += mwords;
            ++ns;
        } else {
            voff += dense;
        }
    }
    sizes->values_bytes = (uint64_t)elem_bytes(d->dtype) * voff;
    sizes->meta_bytes = 4 * moff;
    sizes->index_bytes = 16 * (uint64_t)T;
    sizes->n_sparse = ns;
    return ok();
}

hts_status hts_pack(const hts_desc* d, const hts_tile* index, const void* W, int64_t ldw, const float* col_scale,
                    void* values, uint32_t* meta, void* stream) {
    hts_status st = check_desc(d);
    if (st) return st;
    if ((st = check_ptr(index, "index")) || (st = check_ptr(W, "W")) || (st = check_ptr(values, "values")))
        return st;
    if (meta && !aligned16(meta)) return fail(HTS_ERR_ALIGN, "meta is not 16-byte aligned");
    if (col_scale && (reinterpret_cast<uintptr_t>(col_scale) & 3u))
        return fail(HTS_ERR_ALIGN, "col_scale is not 4-byte aligned");
    if ((st = check_ld(ldw, d->K, ld_mult(d->dtype), "ldw"))) return st;
    if (debug_mode() &&
        ((st = debug_packed(d, index, values, meta, static_cast<hipStream_t>(stream), true)) ||
         (st = debug_range(W, block_bytes(d->N, d->K, ldw, elem_bytes(d->dtype)), "W")) ||
         (st = debug_range(col_scale, 4 * (uint64_t)d->K, "col_scale"))))
        return st;
    return hip_status(hts::launch_pack(*d, index, static_cast<const uint16_t*>(W), ldw, col_scale,
                                       static_cast<uint16_t*>(values), meta, static_cast<hipStream_t>(stream)),
                      "pack kernel launch");
}

hts_status hts_pack_masked(const hts_desc* d, const hts_tile* index, const void* W, int64_t ldw,
                           const uint8_t* mask, int64_t ldm, void* values, uint32_t* meta,
                           uint32_t* malformed_groups, void* stream) {
    hts_status st = check_desc(d);
    if (st) return st;
    if ((st = check_ptr(index, "index")) || (st = check_ptr(W, "W")) || (st = check_ptr(values, "values")) ||
        (st = check_ptr(mask, "mask")))
        return st;
    if (meta && !aligned16(meta)) return fail(HTS_ERR_ALIGN, "meta is not 16-byte aligned");
    if (malformed_groups && (reinterpret_cast<uintptr_t>(malformed_groups) & 3u))
        return fail(HTS_ERR_ALIGN, "malformed_groups is not 4-byte aligned");
    if ((st = check_ld(ldw, d->K, ld_mult(d->dtype), "ldw"))) return st;
    if ((st = check_ld(ldm, d->K, 16, "ldm"))) return st;
    if (debug_mode() &&
        ((st = debug_packed(d, index, values, meta, static_cast<hipStream_t>(stream), true)) ||
         (st = debug_range(W, block_bytes(d->N, d->K, ldw, elem_bytes(d->dtype)), "W")) ||
         (st = debug_range(mask, block_bytes(d->N, d->K, ldm, 1), "mask")) ||
         (st = debug_range(malformed_groups, 4, "malformed_groups"))))
        return st;
    return hip_status(hts::launch_pack_masked(*d, index, static_cast<const uint16_t*>(W), ldw, mask, ldm,
                                              malformed_groups, static_cast<uint16_t*>(values), meta,
                                              static_cast<hipStream_t>(stream)),
                      "masked pack kernel launch");
}

hts_status hts_unpack(const hts_desc* d, const hts_tile* index, const void* values, const uint32_t* meta,
                      void* W_out, int64_t ldw, void* stream) {
    hts_status st = check_desc(d);
    if (st) return st;
    if ((st = check_ptr(index, "index")) || (st = check_ptr(values, "values")) || (st = check_ptr(W_out, "W_out")))
        return st;
    if (meta && !aligned16(meta)) return fail(HTS_ERR_ALIGN, "meta is not 16-byte aligned");
    if ((st = check_ld(ldw, d->K, ld_mult(d->dtype), "ldw"))) return st;
    if (debug_mode() &&
        ((st = debug_packed(d, index, values, meta, static_cast<hipStream_t>(stream), false)) ||
         (st = debug_range(W_out, block_bytes(d->N, d->K, ldw, elem_bytes(d->dtype)), "W_out"))))
        return st;
    return hip_status(hts::launch_unpack(*d, index, static_cast<const uint16_t*>(values), meta,
                                         static_cast<uint16_t*>(W_out), ldw, static_cast<hipStream_t>(stream)),
                      "unpack kernel launch");
}

hts_status hts_gemm_workspace(const hts_desc* d, int64_t M, size_t* bytes) {
    hts_status st = check_desc(d);
    if (st) return st;
    if (M < 0) return fail(HTS_ERR_SHAPE, "M=%lld is negative", (long long)M);
    if (!bytes) return fail(HTS_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = (size_t)gemm_workspace_bytes(d, M);
    return ok();
}

hts_status hts_gemm(const hts_desc* d, const hts_tile* index, const void* values, const uint32_t* meta, int64_t M,
                    const void* X, int64_t ldx, void* Y, int64_t ldy, int32_t y_dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return gemm_impl(d, index, values, meta, M, X, ldx, nullptr, 0, Y, ldy, y_dtype, workspace, workspace_bytes,
                     stream);
}

hts_status hts_gemm_noalloc(const hts_desc* d, const hts_tile* index, const void* values, const uint32_t* meta,
                            int64_t M, const void* X, int64_t ldx, void* Y, int64_t ldy, int32_t y_dtype,
                            void* stream) {
    hts_status st = check_desc(d);
    if (st) return st;
    if (M < 0) return fail(HTS_ERR_SHAPE, "M=%lld is negative", (long long)M);
    const uint64_t need = gemm_workspace_bytes(d, M);
    if (need > kScratchBytes)
        return fail(HTS_ERR_WORKSPACE, "M=%lld on this weight needs %llu bytes of scratch, above the %zu-byte maximum "
                    "of hts_gemm_noalloc (use hts_gemm with a workspace)",
                    (long long)M, (unsigned long long)need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0 && (st = g_scratch.get(&ws))) return st;
    return gemm_impl(d, index, values, meta, M, X, ldx, nullptr, 0, Y, ldy, y_dtype, ws, ws ? kScratchBytes : 0,
                     stream, false);
}

hts_status hts_gemm_silu_mul(const hts_desc* d, const hts_tile* index, const void* values, const uint32_t* meta,
                             int64_t M, const void* X, int64_t ldx, const void* G, int64_t ldg, void* Y, int64_t ldy,
                             int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (M > 0) {
        if (!G) return fail(HTS_ERR_INVALID_ARG, "G is NULL");
        hts_status st = check_ld(ldg, d ? d->N : 0, 4, "ldg");
        if (st) return st;
    }
    return gemm_impl(d, index, values, meta, M, X, ldx, G, ldg, Y, ldy, y_dtype, workspace, workspace_bytes, stream);
}

hts_status hts_dense_gemm(int32_t dtype, int64_t M, int64_t N, int64_t K, const void* X, int64_t ldx, const void* W,
                          int64_t ldw, void* Y, int64_t ldy, int32_t y_dtype, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!is_in(dtype)) return fail(HTS_ERR_DTYPE, "dtype %d is not HTS_F16, HTS_BF16 or HTS_FP8_E4M3", dtype);
    if (!is_out(y_dtype)) return fail(HTS_ERR_DTYPE, "y_dtype %d is not F32, F16 or BF16", y_dtype);
    if (M < 0 || N <= 0 || K <= 0)
        return fail(HTS_ERR_SHAPE, "M=%lld N=%lld K=%lld (M >= 0, N and K positive)", (long long)M, (long long)N,
                    (long long)K);
    if (N % 64 || K % 64) return fail(HTS_ERR_SHAPE, "N and K must be multiples of 64");
    if (dtype == HTS_FP8_E4M3 && (N % 128 || K % 128))
        return fail(HTS_ERR_SHAPE, "8-bit products need N and K multiples of 128");
    hts_status st;
    const int lm = ld_mult(dtype);
    if ((st = check_ld(ldx, K, lm, "ldx")) || (st = check_ld(ldw, K, lm, "ldw")) || (st = check_ld(ldy, N, 4, "ldy")))
        return st;
    if (M == 0) return ok();
    if ((st = check_ptr(X, "X")) || (st = check_ptr(W, "W")) || (st = check_ptr(Y, "Y"))) return st;
    if (workspace && !aligned16(workspace)) return fail(HTS_ERR_ALIGN, "workspace is not 16-byte aligned");
    if (debug_mode() &&
        ((st = debug_range(X, block_bytes(M, K, ldx, elem_bytes(dtype)), "X")) ||
         (st = debug_range(W, block_bytes(N, K, ldw, elem_bytes(dtype)), "W")) ||
         (st = debug_range(Y, block_bytes(M, N, ldy, y_dtype == HTS_F32 ? 4 : 2), "Y")) ||
         (st = debug_range(workspace, workspace_bytes, "workspace"))))
        return st;
    hts::GemmArgs a{};
    a.dtype = dtype;
    a.y_dtype = y_dtype;
    a.M = M;
    a.N = N;
    a.K = K;
    a.bn = 64;
    a.bk = (K % 128 == 0) ? 128 : 64;
    a.W = static_cast<const uint16_t*>(W);
    a.ldw = ldw;
    a.X = static_cast<const uint16_t*>(X);
    a.ldx = ldx;
    a.Y = Y;
    a.ldy = ldy;
    attach_split(a, prefill_split(M, N, K, dtype, a.bk, 128), workspace, workspace_bytes);
    return run_gemm(a, static_cast<hipStream_t>(stream));
}

hts_status hts_dense_gemm_workspace(int32_t dtype, int64_t M, int64_t N, int64_t K, size_t* bytes) {
    if (!is_in(dtype)) return fail(HTS_ERR_DTYPE, "dtype %d is not HTS_F16, HTS_BF16 or HTS_FP8_E4M3", dtype);
    if (M < 0 || N <= 0 || K <= 0)
        return fail(HTS_ERR_SHAPE, "M=%lld N=%lld K=%lld (M >= 0, N and K positive)", (long long)M, (long long)N,
                    (long long)K);
    if (!bytes) return fail(HTS_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = (size_t)split_bytes(M, N, prefill_split(M, N, K, dtype, (K % 128 == 0) ? 128 : 64, 128));
    return ok();
}

hts_status hts_silu_mul(int32_t dtype, int64_t M, int64_t N, const void* G, int64_t ldg, const void* U,
                        int64_t ldu, void* H, int64_t ldh, void* stream) {
    if (dtype != HTS_F16 && dtype != HTS_BF16) return fail(HTS_ERR_DTYPE, "dtype %d is not F16 or BF16", dtype);
    if (M < 0 || N <= 0) return fail(HTS_ERR_SHAPE, "M=%lld N=%lld (M >= 0, N positive)", (long long)M, (long long)N);
    if (N % 8) return fail(HTS_ERR_SHAPE, "N=%lld is not a multiple of 8", (long long)N);
    if (M == 0) return ok();
    hts_status st;
    if ((st = check_ptr(G, "G")) || (st = check_ptr(U, "U")) || (st = check_ptr(H, "H"))) return st;
    if ((st = check_ld(ldg, N, 8, "ldg")) || (st = check_ld(ldu, N, 8, "ldu")) || (st = check_ld(ldh, N, 8, "ldh")))
        return st;
    if (debug_mode() && ((st = debug_range(G, block_bytes(M, N, ldg, 2), "G")) ||
                         (st = debug_range(U, block_bytes(M, N, ldu, 2), "U")) ||
                         (st = debug_range(H, block_bytes(M, N, ldh, 2), "H"))))
        return st;
    return hip_status(hts::launch_silu_mul(dtype, M, N, static_cast<const uint16_t*>(G), ldg,
                                           static_cast<const uint16_t*>(U), ldu, static_cast<uint16_t*>(H), ldh,
                                           static_cast<hipStream_t>(stream)),
                      "silu_mul kernel launch");
}

hts_status hts_col_norms(int32_t dtype, int64_t rows, int64_t K, const void* X, int64_t ldx, float* col_scale,
                         void* stream) {
    if (!is16bit(dtype)) return fail(HTS_ERR_DTYPE, "dtype %d is not HTS_F16 or HTS_BF16", dtype);
    if (rows <= 0 || K <= 0) return fail(HTS_ERR_SHAPE, "rows and K must be positive");
    hts_status st;
    if ((st = check_ld(ldx, K, 1, "ldx"))) return st;
    if (!X || !col_scale) return fail(HTS_ERR_INVALID_ARG, "X or col_scale is NULL");
    if ((reinterpret_cast<uintptr_t>(X) & 1u) || (reinterpret_cast<uintptr_t>(col_scale) & 3u))
        return fail(HTS_ERR_ALIGN, "X must be 2-byte and col_scale 4-byte aligned");
    if (debug_mode() && ((st = debug_range(X, block_bytes(rows, K, ldx, 2), "X")) ||
                         (st = debug_range(col_scale, 4 * (uint64_t)K, "col_scale"))))
        return st;
    return hip_status(hts::launch_col_norms(dtype, rows, K, static_cast<const uint16_t*>(X), ldx, col_scale,
                                            static_cast<hipStream_t>(stream)),
                      "column-norm kernel launch");
}

hts_status hts_wanda_tile_cost(const hts_desc* d, const void* W, int64_t ldw, const float* col_scale, double* cost,
                               void* stream) {
    hts_status st = check_desc(d);
    if (st) return st;
    if (!is16bit(d->dtype)) return fail(HTS_ERR_DTYPE, "tile costs take HTS_F16 or HTS_BF16 weights");
    if ((st = check_ptr(W, "W")) || (st = check_ld(ldw, d->K, 8, "ldw"))) return st;
    if (!col_scale || !cost) return fail(HTS_ERR_INVALID_ARG, "col_scale or cost is NULL");
    if ((reinterpret_cast<uintptr_t>(col_scale) & 3u) || (reinterpret_cast<uintptr_t>(cost) & 7u))
        return fail(HTS_ERR_ALIGN, "col_scale must be 4-byte and cost 8-byte aligned");
    if (debug_mode() && ((st = debug_range(W, block_bytes(d->N, d->K, ldw, 2), "W")) ||
                         (st = debug_range(col_scale, 4 * (uint64_t)d->K, "col_scale")) ||
                         (st = debug_range(cost, 8 * (uint64_t)((d->N / d->bn) * (d->K / d->bk)), "cost"))))
        return st;
    return hip_status(hts::launch_wanda_cost(*d, static_cast<const uint16_t*>(W), ldw, col_scale, cost,
                                             static_cast<hipStream_t>(stream)),
                      "tile-cost kernel launch");
}

hts_status hts_wanda_map(int64_t T, const double* cost, int64_t n_sparse, uint8_t* map, void* stream) {
    if (T <= 0) return fail(HTS_ERR_SHAPE, "T must be positive");
    if (n_sparse < 0 || n_sparse > T) return fail(HTS_ERR_SHAPE, "n_sparse=%lld outside 0..T", (long long)n_sparse);
    if (!cost || !map) return fail(HTS_ERR_INVALID_ARG, "cost or map is NULL");
    if (reinterpret_cast<uintptr_t>(cost) & 7u) return fail(HTS_ERR_ALIGN, "cost must be 8-byte aligned");
    hts_status st;
    if (debug_mode() && ((st = debug_range(cost, 8 * (uint64_t)T, "cost")) || (st = debug_range(map, (uint64_t)T, "map"))))
        return st;
    return hip_status(hts::launch_wanda_map(T, cost, n_sparse, map, static_cast<hipStream_t>(stream)),
                      "tile-map kernel launch");
}

}  // extern "C"
