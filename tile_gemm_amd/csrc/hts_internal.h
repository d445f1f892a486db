// Internal declarations shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "hts.h"

namespace hts {

// A host-side action done once per device (e.g. raising a kernel's dynamic-LDS limit, which
// applies to the current device): thread-safe, retried on a later call if it failed.
class DeviceOnce {
  public:
    static constexpr int kMaxDevices = 64;
    template <typename F>
    hipError_t run(F&& f) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
        if (done_[dev].load(std::memory_order_acquire)) return hipSuccess;
        std::lock_guard<std::mutex> lock(mu_);
        if (done_[dev].load(std::memory_order_relaxed)) return hipSuccess;
        e = f();
        if (e == hipSuccess) done_[dev].store(true, std::memory_order_release);
        return e;
    }

  private:
    std::mutex mu_;
    std::atomic<bool> done_[kMaxDevices] = {};
};

// Everything a product kernel needs, by value.  Exactly one weight source is
// used: the packed hybrid weight (index/values/meta) or a row-major W (W/ldw).
struct GemmArgs {
    int32_t dtype;        // HTS_F16 / HTS_BF16 for X and W
    int32_t y_dtype;      // HTS_F32 / HTS_F16 / HTS_BF16
    int64_t M, N, K;
    int32_t bn, bk;       // tile size (a row-major W uses a virtual grid of bn x bk)
    const hts_tile* index;
    const uint16_t* values;
    const uint32_t* meta;
    const uint16_t* W;    // row-major weight (dense product) or nullptr
    int64_t ldw;
    const uint16_t* X;
    int64_t ldx;
    void* Y;
    int64_t ldy;
    // tiled kernel only: nsplit > 1 splits each tile row's slices over nsplit workgroups, which
    // write fp32 partial products to part[nsplit][M][N]; a reduction then writes Y
    float* part;
    int32_t nsplit;
    // gated output (hts_gemm_silu_mul): Y = silu(G) * (X . W^T), G[M,N] (ldg) in y_dtype, or nullptr
    const void* gate;
    int64_t ldg;
};

enum SparsePath { SPARSE_SMFMAC = 0, SPARSE_DECOMPRESS = 1 };

hipError_t launch_pack(const hts_desc& d, const hts_tile* index, const uint16_t* W, int64_t ldw,
                       const float* col_scale, uint16_t* values, uint32_t* meta, hipStream_t s);
// mask: uint8 [N, ldm], nonzero = keep (read in 2:4 tiles only); malformed: counter or nullptr
hipError_t launch_pack_masked(const hts_desc& d, const hts_tile* index, const uint16_t* W, int64_t ldw,
                              const uint8_t* mask, int64_t ldm, uint32_t* malformed, uint16_t* values,
                              uint32_t* meta, hipStream_t s);
hipError_t launch_unpack(const hts_desc& d, const hts_tile* index, const uint16_t* values,
                         const uint32_t* meta, uint16_t* W_out, int64_t ldw, hipStream_t s);
// Debug check of a device tile index (HTS_DEBUG=1): `out` must hold {0, 0xFFFFFFFF, 0, 0} before
// the launch; afterwards bad = inconsistent records, first_bad = the first of them, and
// values_end / meta_end = where the last tile's values (elements) and codes (words) end.
struct IndexCheck {
    uint32_t bad, first_bad;
    uint64_t values_end, meta_end;
};
hipError_t launch_index_check(const hts_desc& d, const hts_tile* index, IndexCheck* out, hipStream_t s);
// ksplit: waves per workgroup (4, 8 or 16); nt: 128-wide tile columns per batch of loads (2 or 4);
// pp: 16-row panels per workgroup (1 or 2; 2 requires N % 32 == 0)
hipError_t launch_gemm_decode(const GemmArgs& a, int ksplit, int nt, int pp, int sparse_path, hipStream_t s);
// Tiled kernel (128 weight rows -- one 128-row tile row or two 64-row ones -- x 64, 128 or 192 X
// rows per workgroup); with a.nsplit > 1 it also launches the fixed-order sum of the partial
// products into Y.
hipError_t launch_gemm_prefill(const GemmArgs& a, int sparse_path, hipStream_t s);
// X rows per block of the tiled kernel (64, 128 or 192) for M rows of X, N weight rows in blocks
// of block_rows (128 or 64); the split planner counts blocks with it.
int prefill_block_m(int64_t M, int64_t N, int32_t dtype, int block_rows);
// Weight rows per block of the tiled kernel on a packed weight with bn-row tiles (16-bit data).
int prefill_weight_rows(int bn);
// With a packed weight and M above the streaming range, K / bk must not exceed this: the
// tiled kernel holds the index records of a block's tile rows in LDS.
constexpr int kMaxTileColsPerRow = 256;
hipError_t launch_silu_mul(int32_t dtype, int64_t M, int64_t N, const uint16_t* G, int64_t ldg, const uint16_t* U,
                           int64_t ldu, uint16_t* H, int64_t ldh, hipStream_t s);
hipError_t launch_col_norms(int32_t dtype, int64_t rows, int64_t K, const uint16_t* X, int64_t ldx,
                            float* out, hipStream_t s);
hipError_t launch_wanda_cost(const hts_desc& d, const uint16_t* W, int64_t ldw, const float* cs,
                             double* cost, hipStream_t s);
hipError_t launch_wanda_map(int64_t T, const double* cost, int64_t n_sparse, uint8_t* map,
                            hipStream_t s);

}  // namespace hts
