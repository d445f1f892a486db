// Stand-ins for the kernel launchers, for a host-only build of the C API under AddressSanitizer
// and UndefinedBehaviorSanitizer (test infrastructure: no GPU code, nothing is launched).  Each
// records the call and checks what the host code hands to the kernels: workspace pointers and
// sizes inside the buffer the caller gave, launch-shape parameters in their documented ranges.
#include <cstdio>
#include <cstdlib>

#include "hts.h"
#include "hts_internal.h"
#include "stub_log.h"

namespace stub {
Log g;
void complain(const char* what) {
    ++g.bad;
    std::fprintf(stderr, "stub check failed: %s\n", what);
}
static bool in_workspace(const void* p, uint64_t bytes) {
    const char* lo = static_cast<const char*>(g.ws);
    const char* q = static_cast<const char*>(p);
    return lo && q >= lo && q + bytes <= lo + g.ws_bytes;
}
}  // namespace stub

namespace hts {
using stub::complain;
using stub::g;

hipError_t launch_pack(const hts_desc& d, const hts_tile* index, const uint16_t* W, int64_t ldw, const float*,
                       uint16_t* values, uint32_t*, hipStream_t) {
    ++g.pack;
    if (!index || !W || !values || ldw < d.K) complain("pack arguments");
    return hipSuccess;
}
hipError_t launch_pack_masked(const hts_desc& d, const hts_tile* index, const uint16_t* W, int64_t ldw,
                              const uint8_t* mask, int64_t ldm, uint32_t*, uint16_t* values, uint32_t*,
                              hipStream_t) {
    ++g.pack_masked;
    if (!index || !W || !mask || !values || ldw < d.K || ldm < d.K) complain("masked pack arguments");
    return hipSuccess;
}
hipError_t launch_index_check(const hts_desc&, const hts_tile* index, IndexCheck* out, hipStream_t) {
    if (!index || !out) complain("index check arguments");
    return hipSuccess;
}
hipError_t launch_unpack(const hts_desc& d, const hts_tile* index, const uint16_t* values, const uint32_t*,
                         uint16_t* W_out, int64_t ldw, hipStream_t) {
    ++g.unpack;
    if (!index || !values || !W_out || ldw < d.K) complain("unpack arguments");
    // the unpack into a product's workspace must fit in it
    if (g.expect_unpack_ws &&
        !stub::in_workspace(W_out, (uint64_t)d.N * ldw * (d.dtype == HTS_FP8_E4M3 ? 1 : 2)))
        complain("unpacked weight outside the workspace");
    return hipSuccess;
}
static void check_gemm(const GemmArgs& a) {
    if (a.M <= 0 || a.N <= 0 || a.K <= 0 || !a.X || !a.Y) complain("product shape or operands");
    if ((a.index == nullptr) == (a.W == nullptr)) complain("exactly one weight source");
    if (a.ldx < a.K || a.ldy < a.N) complain("leading dimensions");
    if (a.nsplit > 1) {
        if (!a.part) complain("split product without parts");
        else if (!stub::in_workspace(a.part, (uint64_t)a.nsplit * a.M * a.N * 4)) complain("split parts outside the workspace");
    }
    g.last_nsplit = a.nsplit;
}
hipError_t launch_gemm_decode(const GemmArgs& a, int ksplit, int nt, int pp, int sparse_path, hipStream_t) {
    ++g.decode;
    check_gemm(a);
    if (!(ksplit == 4 || ksplit == 8 || ksplit == 16) || !(nt == 1 || nt == 2 || nt == 4) || !(pp == 1 || pp == 2) ||
        !(sparse_path == 0 || sparse_path == 1))
        complain("streaming launch shape");
    if (pp == 2 && a.N % 32) complain("two panels need N % 32 == 0");
    return hipSuccess;
}
hipError_t launch_gemm_prefill(const GemmArgs& a, int sparse_path, hipStream_t) {
    ++g.prefill;
    check_gemm(a);
    if (!(sparse_path == 0 || sparse_path == 1)) complain("sparse path");
    return hipSuccess;
}
// the split planner's block height (the kernel side's rule, restated)
int prefill_block_m(int64_t M, int64_t N, int32_t dtype, int block_rows) {
    if (M <= 64) return dtype == HTS_FP8_E4M3 ? 128 : 64;
    if (block_rows != 128) return 128;
    const int64_t nb = (N + 127) / 128, b128 = nb * ((M + 127) / 128), b192 = nb * ((M + 191) / 192);
    if (b128 <= 256) return 128;
    return ((b192 + 511) / 512) * 139 < ((b128 + 511) / 512) * 97 ? 192 : 128;
}
// weight rows per block on 64-row tiles (the kernel side's rule, restated): two tile rows
int prefill_weight_rows(int bn) {
    if (bn != 64) return 128;
    const char* v = getenv("HTS_PREFILL_TWO_ROWS");
    return (v && v[0] == '0' && !v[1]) ? 64 : 128;
}
hipError_t launch_silu_mul(int32_t, int64_t M, int64_t N, const uint16_t* G, int64_t ldg, const uint16_t* U,
                           int64_t ldu, uint16_t* H, int64_t ldh, hipStream_t) {
    ++g.silu;
    if (M <= 0 || N <= 0 || !G || !U || !H || ldg < N || ldu < N || ldh < N) complain("silu_mul arguments");
    return hipSuccess;
}
hipError_t launch_col_norms(int32_t, int64_t rows, int64_t K, const uint16_t* X, int64_t ldx, float* out,
                            hipStream_t) {
    ++g.col_norms;
    if (rows <= 0 || K <= 0 || !X || !out || ldx < K) complain("col_norms arguments");
    return hipSuccess;
}
hipError_t launch_wanda_cost(const hts_desc& d, const uint16_t* W, int64_t ldw, const float* cs, double* cost,
                             hipStream_t) {
    ++g.wanda_cost;
    if (!W || !cs || !cost || ldw < d.K) complain("wanda cost arguments");
    return hipSuccess;
}
hipError_t launch_wanda_map(int64_t T, const double* cost, int64_t n_sparse, uint8_t* map, hipStream_t) {
    ++g.wanda_map;
    if (T <= 0 || !cost || !map || n_sparse < 0 || n_sparse > T) complain("wanda map arguments");
    return hipSuccess;
}
}  // namespace hts
