// Host-only driver of the C API for the AddressSanitizer / UndefinedBehaviorSanitizer build (test
// infrastructure).  The kernel launchers are stand-ins (launch_stubs.cpp), so every entry point
// runs its argument checks, tile-index planning, workspace arithmetic and launch-shape choice on
// the host, and the sanitizers watch that code.  "Device" buffers are host memory that the host
// code never dereferences.  Exit status 0 = every expectation held and the stubs saw no bad
// arguments.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "hts.h"
#include "stub_log.h"

static std::atomic<int> fails{0};
#define EXPECT(cond, ...)                                                   \
    do {                                                                    \
        if (!(cond)) {                                                      \
            ++fails;                                                        \
            std::fprintf(stderr, "FAIL line %d: ", __LINE__);               \
            std::fprintf(stderr, __VA_ARGS__);                              \
            std::fprintf(stderr, "  [%s]\n", hts_last_error());             \
        }                                                                   \
    } while (0)

static hts_desc desc(int64_t N, int64_t K, int bn, int bk, int dt) { return hts_desc{N, K, bn, bk, dt, 0}; }

// host stand-in for device memory: 16-byte (and 256-byte) aligned, never dereferenced
alignas(256) static unsigned char fake[1 << 16];
static void* dev(size_t off = 0) { return fake + off; }

static void test_plan(std::mt19937& rng) {
    const int dts[3] = {HTS_F16, HTS_BF16, HTS_FP8_E4M3};
    const int tiles[3] = {32, 64, 128};
    for (int dt : dts)
        for (int bn : tiles)
            for (int bk : tiles) {
                if (dt == HTS_FP8_E4M3 && (bn != 128 || bk != 128)) {
                    hts_desc d = desc(256, 256, bn, bk, dt);
                    uint8_t m[64] = {};
                    hts_sizes s;
                    EXPECT(hts_pack_plan(&d, m, nullptr, &s) == HTS_ERR_UNSUPPORTED, "fp8 %dx%d", bn, bk);
                    continue;
                }
                for (int trial = 0; trial < 4; ++trial) {
                    const int64_t N = bn * (1 + (int64_t)(rng() % 9)), K = bk * (1 + (int64_t)(rng() % 9));
                    const int64_t T = (N / bn) * (K / bk);
                    std::vector<uint8_t> map((size_t)T);
                    const unsigned p = trial;   // 0: all dense, 3: all 2:4, else mixed
                    for (auto& v : map) v = p == 0 ? 0 : p == 3 ? 1 : (uint8_t)(rng() & 1);
                    std::unique_ptr<hts_tile[]> index(new hts_tile[(size_t)T]);   // exactly T records
                    hts_desc d = desc(N, K, bn, bk, dt);
                    hts_sizes s{}, q{};
                    EXPECT(hts_pack_plan(&d, map.data(), index.get(), &s) == HTS_OK, "plan %lldx%lld", (long long)N,
                           (long long)K);
                    EXPECT(hts_last_error()[0] == '\0', "error text after success");
                    EXPECT(hts_pack_plan(&d, map.data(), nullptr, &q) == HTS_OK, "sizes only");
                    EXPECT(std::memcmp(&s, &q, sizeof s) == 0, "sizes differ with and without the index");
                    const uint64_t es = dt == HTS_FP8_E4M3 ? 1 : 2, dense = (uint64_t)bn * bk;
                    uint64_t v = 0, m = 0;
                    int64_t ns = 0;
                    for (int64_t t = 0; t < T; ++t) {
                        EXPECT(index[t].val_off == v && index[t].meta_off == m && index[t].type == map[t] &&
                                   index[t].reserved == 0,
                               "record %lld", (long long)t);
                        v += map[t] ? dense / 2 : dense;
                        m += map[t] ? dense / 32 : 0;
                        ns += map[t];
                    }
                    EXPECT(s.values_bytes == es * v && s.meta_bytes == 4 * m && s.index_bytes == 16 * (uint64_t)T &&
                               s.n_sparse == ns,
                           "sizes");
                    map[(size_t)(rng() % T)] = (uint8_t)(2 + rng() % 250);
                    EXPECT(hts_pack_plan(&d, map.data(), index.get(), &s) == HTS_ERR_MAP, "bad map entry");
                }
            }
    // the largest grid below 2^32 weights (the index of 261,632 tiles is filled), then one past it
    {
        hts_desc d = desc(65536, 65408, 128, 128, HTS_BF16);
        const int64_t T = (65536 / 128) * (65408 / 128);
        std::vector<uint8_t> map((size_t)T, 1);
        std::unique_ptr<hts_tile[]> index(new hts_tile[(size_t)T]);
        hts_sizes s{};
        EXPECT(hts_pack_plan(&d, map.data(), index.get(), &s) == HTS_OK, "largest grid");
        EXPECT(index[T - 1].val_off == (uint64_t)(T - 1) * 128 * 64, "last offset");
        hts_desc e = desc(65536, 65536, 128, 128, HTS_BF16);
        EXPECT(hts_pack_plan(&e, map.data(), nullptr, &s) == HTS_ERR_SHAPE, "N*K = 2^32");
    }
}

static void test_descriptors() {
    uint8_t map[64] = {};
    hts_sizes s;
    struct Case { hts_desc d; int want; } cases[] = {
        {desc(256, 256, 128, 128, HTS_F32), HTS_ERR_DTYPE},
        {desc(256, 256, 128, 128, 7), HTS_ERR_DTYPE},
        {desc(256, 256, 128, 128, -1), HTS_ERR_DTYPE},
        {desc(0, 256, 128, 128, HTS_BF16), HTS_ERR_SHAPE},
        {desc(256, -128, 128, 128, HTS_BF16), HTS_ERR_SHAPE},
        {desc(256, 256, 16, 128, HTS_BF16), HTS_ERR_UNSUPPORTED},
        {desc(256, 256, 128, 256, HTS_BF16), HTS_ERR_UNSUPPORTED},
        {desc(256, 256, 0, 0, HTS_BF16), HTS_ERR_UNSUPPORTED},
        {desc(200, 256, 128, 128, HTS_BF16), HTS_ERR_SHAPE},
        {desc(256, 192, 128, 128, HTS_BF16), HTS_ERR_SHAPE},
        {desc(256, 256, 64, 64, HTS_FP8_E4M3), HTS_ERR_UNSUPPORTED},
        {desc(INT64_MAX / 2, 128, 128, 128, HTS_BF16), HTS_ERR_SHAPE},
    };
    for (auto& c : cases) EXPECT(hts_pack_plan(&c.d, map, nullptr, &s) == c.want, "descriptor -> %d", c.want);
    hts_desc r = desc(256, 256, 128, 128, HTS_BF16);
    r.reserved = 1;
    EXPECT(hts_pack_plan(&r, map, nullptr, &s) == HTS_ERR_INVALID_ARG, "reserved field");
    EXPECT(hts_pack_plan(nullptr, map, nullptr, &s) == HTS_ERR_INVALID_ARG, "null descriptor");
    hts_desc d = desc(256, 256, 128, 128, HTS_BF16);
    EXPECT(hts_pack_plan(&d, nullptr, nullptr, &s) == HTS_ERR_INVALID_ARG, "null map");
    EXPECT(hts_pack_plan(&d, map, nullptr, nullptr) == HTS_ERR_INVALID_ARG, "null sizes");
    for (int code : {-1, 0, 1, 8, 9, 99, -2147483647 - 1}) EXPECT(hts_status_string(code) != nullptr, "status %d", code);
    EXPECT(hts_abi_version() == HTS_ABI_VERSION, "abi version");
}

static void test_pack_unpack() {
    hts_desc d = desc(256, 512, 128, 128, HTS_BF16);
    const hts_tile* idx = static_cast<const hts_tile*>(dev());
    const int before = stub::g.pack + stub::g.pack_masked + stub::g.unpack;
    EXPECT(hts_pack(&d, idx, dev(), 512, nullptr, dev(4096), static_cast<uint32_t*>(dev(8192)), nullptr) == HTS_OK,
           "pack");
    EXPECT(hts_pack(&d, idx, dev(), 511, nullptr, dev(4096), nullptr, nullptr) == HTS_ERR_SHAPE, "pack ldw < K");
    EXPECT(hts_pack(&d, idx, dev(), 514, nullptr, dev(4096), nullptr, nullptr) == HTS_ERR_ALIGN, "pack ldw not a multiple of 8");
    EXPECT(hts_pack(&d, idx, dev(2), 512, nullptr, dev(4096), nullptr, nullptr) == HTS_ERR_ALIGN, "pack W align");
    EXPECT(hts_pack(&d, nullptr, dev(), 512, nullptr, dev(4096), nullptr, nullptr) == HTS_ERR_INVALID_ARG, "pack index");
    EXPECT(hts_pack(&d, idx, dev(), 512, static_cast<const float*>(dev(2)), dev(4096), nullptr, nullptr) ==
               HTS_ERR_ALIGN,
           "pack col_scale align");
    EXPECT(hts_pack(&d, idx, dev(), 512, nullptr, dev(4096), static_cast<uint32_t*>(dev(8196)), nullptr) ==
               HTS_ERR_ALIGN,
           "pack meta align");
    EXPECT(hts_pack_masked(&d, idx, dev(), 512, static_cast<const uint8_t*>(dev(1024)), 512, dev(4096),
                           static_cast<uint32_t*>(dev(8192)), static_cast<uint32_t*>(dev(12288)), nullptr) == HTS_OK,
           "masked pack");
    EXPECT(hts_pack_masked(&d, idx, dev(), 512, static_cast<const uint8_t*>(dev(1024)), 500, dev(4096), nullptr,
                           nullptr, nullptr) == HTS_ERR_SHAPE,
           "masked pack ldm");
    EXPECT(hts_pack_masked(&d, idx, dev(), 512, nullptr, 512, dev(4096), nullptr, nullptr, nullptr) ==
               HTS_ERR_INVALID_ARG,
           "masked pack mask");
    EXPECT(hts_unpack(&d, idx, dev(4096), nullptr, dev(), 512, nullptr) == HTS_OK, "unpack");
    EXPECT(hts_unpack(&d, idx, dev(4096), nullptr, nullptr, 512, nullptr) == HTS_ERR_INVALID_ARG, "unpack W_out");
    EXPECT(hts_unpack(&d, idx, dev(4096), nullptr, dev(), 256, nullptr) == HTS_ERR_SHAPE, "unpack ldw");
    EXPECT(stub::g.pack + stub::g.pack_masked + stub::g.unpack == before + 3, "launch count %d",
           stub::g.pack + stub::g.pack_masked + stub::g.unpack - before);
}

// Workspace: exactly what hts_gemm_workspace asks for, in host memory; the stubs check that every
// part the product uses lies inside it.
static void run_gemm_case(const hts_desc& d, int64_t M, bool give_workspace) {
    size_t need = 0;
    EXPECT(hts_gemm_workspace(&d, M, &need) == HTS_OK, "workspace query M=%lld", (long long)M);
    std::unique_ptr<unsigned char[]> buf(need ? new unsigned char[need + 256] : nullptr);
    void* ws = nullptr;
    if (need && give_workspace) ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(buf.get()) + 255) & ~uintptr_t(255));
    stub::g.ws = ws;
    stub::g.ws_bytes = ws ? need : 0;
    stub::g.expect_unpack_ws = true;
    const int64_t ldx = d.K, ldy = d.N;
    const int launches = stub::g.decode + stub::g.prefill;
    stub::g.last_nsplit = 0;
    const hts_status st = hts_gemm(&d, static_cast<const hts_tile*>(dev()), dev(), static_cast<const uint32_t*>(dev()), M,
                                   dev(), ldx, dev(), ldy, HTS_BF16, ws, ws ? need : 0, nullptr);
    const bool small = d.bn < 64 || d.bk < 64;
    if (need && !give_workspace && small) {
        EXPECT(st == HTS_ERR_WORKSPACE, "32-wide tiles without workspace M=%lld", (long long)M);
    } else {
        EXPECT(st == HTS_OK, "gemm M=%lld tile %dx%d", (long long)M, d.bn, d.bk);
        EXPECT(stub::g.decode + stub::g.prefill == launches + (M > 0 ? 1 : 0), "one product launch (none at M = 0)");
        if (!ws) EXPECT(stub::g.last_nsplit <= 1, "split without workspace");
    }
    // the gated product: the same planning, G checked
    if (ws || !need) {
        EXPECT(hts_gemm_silu_mul(&d, static_cast<const hts_tile*>(dev()), dev(), static_cast<const uint32_t*>(dev()), M,
                                 dev(), ldx, dev(), ldy, dev(), ldy, HTS_BF16, ws, ws ? need : 0, nullptr) == HTS_OK,
               "gated M=%lld", (long long)M);
        if (M > 0)
            EXPECT(hts_gemm_silu_mul(&d, static_cast<const hts_tile*>(dev()), dev(), static_cast<const uint32_t*>(dev()),
                                     M, dev(), ldx, nullptr, ldy, dev(), ldy, HTS_BF16, ws, ws ? need : 0, nullptr) ==
                       HTS_ERR_INVALID_ARG,
                   "gated without G");
    }
    stub::g.ws = nullptr;
    stub::g.ws_bytes = 0;
    stub::g.expect_unpack_ws = false;
}

static void test_gemm() {
    const hts_desc shapes[] = {desc(11008, 4096, 128, 128, HTS_BF16), desc(4096, 4096, 64, 64, HTS_F16),
                               desc(1024, 512, 32, 32, HTS_BF16), desc(256, 2048, 128, 128, HTS_FP8_E4M3),
                               desc(512, 384, 64, 128, HTS_BF16)};
    const int64_t Ms[] = {0, 1, 5, 16, 17, 32, 33, 64, 128, 129, 256, 257, 300, 2048};
    for (const auto& d : shapes)
        for (int64_t M : Ms) {
            run_gemm_case(d, M, true);
            run_gemm_case(d, M, false);
        }
    hts_desc d = desc(1024, 512, 128, 128, HTS_BF16);
    const hts_tile* idx = static_cast<const hts_tile*>(dev());
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, -1, dev(), 512, dev(), 1024, HTS_BF16, nullptr, 0, nullptr) ==
               HTS_ERR_SHAPE,
           "negative M");
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 4, dev(), 512, dev(), 1024, 9, nullptr, 0, nullptr) == HTS_ERR_DTYPE,
           "y dtype");
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 4, dev(), 500, dev(), 1024, HTS_BF16, nullptr, 0, nullptr) ==
               HTS_ERR_SHAPE,
           "ldx");
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 4, dev(), 512, dev(), 1022, HTS_BF16, nullptr, 0, nullptr) ==
               HTS_ERR_SHAPE,
           "ldy");
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 4, dev(8), 512, dev(), 1024, HTS_BF16, nullptr, 0, nullptr) ==
               HTS_ERR_ALIGN,
           "X align");
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 4, dev(), 512, nullptr, 1024, HTS_BF16, nullptr, 0, nullptr) ==
               HTS_ERR_INVALID_ARG,
           "Y null");
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 300, dev(), 512, dev(), 1024, HTS_BF16, dev(8), 1 << 20, nullptr) ==
               HTS_ERR_ALIGN,
           "workspace align");
    size_t n = 0;
    EXPECT(hts_gemm_workspace(&d, 4, nullptr) == HTS_ERR_INVALID_ARG, "workspace null out");
    EXPECT(hts_gemm_workspace(&d, -3, &n) == HTS_ERR_SHAPE, "workspace negative M");
    // dense product
    for (int64_t M : Ms) {
        size_t need = 0;
        EXPECT(hts_dense_gemm_workspace(HTS_BF16, M, 11008, 4096, &need) == HTS_OK, "dense workspace");
        std::unique_ptr<unsigned char[]> buf(need ? new unsigned char[need + 256] : nullptr);
        void* ws = need ? reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(buf.get()) + 255) & ~uintptr_t(255)) : nullptr;
        stub::g.ws = ws;
        stub::g.ws_bytes = need;
        EXPECT(hts_dense_gemm(HTS_BF16, M, 11008, 4096, dev(), 4096, dev(), 4096, dev(), 11008, HTS_F32, ws, need,
                              nullptr) == HTS_OK,
               "dense M=%lld", (long long)M);
        stub::g.ws = nullptr;
        stub::g.ws_bytes = 0;
    }
    EXPECT(hts_dense_gemm(HTS_BF16, 4, 100, 4096, dev(), 4096, dev(), 4096, dev(), 100, HTS_F32, nullptr, 0,
                          nullptr) == HTS_ERR_SHAPE,
           "dense N not a multiple of 64");
    EXPECT(hts_dense_gemm(HTS_F32, 4, 128, 128, dev(), 128, dev(), 128, dev(), 128, HTS_F32, nullptr, 0, nullptr) ==
               HTS_ERR_DTYPE,
           "dense dtype");
    EXPECT(hts_dense_gemm(HTS_FP8_E4M3, 4, 192, 128, dev(), 128, dev(), 128, dev(), 192, HTS_F32, nullptr, 0,
                          nullptr) == HTS_ERR_SHAPE,
           "dense fp8 N not a multiple of 128");
    // allocation-free entry point: no scratch needed -> runs; scratch needed -> needs the device
    // (none here: HTS_ERR_HIP), beyond the maximum -> HTS_ERR_WORKSPACE before any device call
    hts_desc b = desc(11008, 4096, 128, 128, HTS_BF16);
    EXPECT(hts_gemm_noalloc(&b, idx, dev(), nullptr, 1, dev(), 4096, dev(), 11008, HTS_BF16, nullptr) == HTS_OK,
           "noalloc M=1");
    const hts_status st = hts_gemm_noalloc(&b, idx, dev(), nullptr, 64, dev(), 4096, dev(), 11008, HTS_BF16, nullptr);
    EXPECT(st == HTS_OK || st == HTS_ERR_HIP, "noalloc M=64 -> %d", (int)st);
    hts_desc big = desc(11008, 4096, 32, 32, HTS_BF16);
    EXPECT(hts_gemm_noalloc(&big, idx, dev(), nullptr, 2048, dev(), 4096, dev(), 11008, HTS_BF16, nullptr) ==
               HTS_ERR_WORKSPACE,
           "noalloc above the scratch maximum");
}

static void test_elementwise_and_wanda() {
    EXPECT(hts_silu_mul(HTS_BF16, 3, 64, dev(), 64, dev(), 64, dev(), 64, nullptr) == HTS_OK, "silu_mul");
    EXPECT(hts_silu_mul(HTS_BF16, 0, 64, nullptr, 64, nullptr, 64, nullptr, 64, nullptr) == HTS_OK, "silu_mul M=0");
    EXPECT(hts_silu_mul(HTS_F32, 3, 64, dev(), 64, dev(), 64, dev(), 64, nullptr) == HTS_ERR_DTYPE, "silu_mul dtype");
    EXPECT(hts_silu_mul(HTS_BF16, 3, 60, dev(), 64, dev(), 64, dev(), 64, nullptr) == HTS_ERR_SHAPE, "silu_mul N not a multiple of 8");
    EXPECT(hts_silu_mul(HTS_BF16, 3, 64, dev(), 56, dev(), 64, dev(), 64, nullptr) == HTS_ERR_SHAPE, "silu_mul ldg");
    EXPECT(hts_col_norms(HTS_BF16, 8, 4096, dev(), 4096, static_cast<float*>(dev(4096)), nullptr) == HTS_OK, "norms");
    EXPECT(hts_col_norms(HTS_BF16, 0, 4096, dev(), 4096, static_cast<float*>(dev(4096)), nullptr) == HTS_ERR_SHAPE,
           "norms rows");
    EXPECT(hts_col_norms(HTS_BF16, 8, 4096, nullptr, 4096, static_cast<float*>(dev(4096)), nullptr) ==
               HTS_ERR_INVALID_ARG,
           "norms X");
    hts_desc d = desc(256, 512, 128, 128, HTS_BF16);
    EXPECT(hts_wanda_tile_cost(&d, dev(), 512, static_cast<const float*>(dev(4096)), static_cast<double*>(dev(8192)),
                               nullptr) == HTS_OK,
           "tile cost");
    hts_desc f8 = desc(256, 512, 128, 128, HTS_FP8_E4M3);
    EXPECT(hts_wanda_tile_cost(&f8, dev(), 512, static_cast<const float*>(dev(4096)), static_cast<double*>(dev(8192)),
                               nullptr) == HTS_ERR_DTYPE,
           "tile cost fp8");
    EXPECT(hts_wanda_tile_cost(&d, dev(), 512, static_cast<const float*>(dev(4096)), static_cast<double*>(dev(8196)),
                               nullptr) == HTS_ERR_ALIGN,
           "tile cost align");
    EXPECT(hts_wanda_map(8, static_cast<const double*>(dev()), 3, static_cast<uint8_t*>(dev(64)), nullptr) == HTS_OK,
           "map");
    EXPECT(hts_wanda_map(8, static_cast<const double*>(dev()), 9, static_cast<uint8_t*>(dev(64)), nullptr) ==
               HTS_ERR_SHAPE,
           "map n_sparse > T");
    EXPECT(hts_wanda_map(0, static_cast<const double*>(dev()), 0, static_cast<uint8_t*>(dev(64)), nullptr) ==
               HTS_ERR_SHAPE,
           "map T = 0");
    EXPECT(hts_wanda_map(8, static_cast<const double*>(dev(4)), 3, static_cast<uint8_t*>(dev(64)), nullptr) ==
               HTS_ERR_ALIGN,
           "map align");
}

// The error text is per thread: threads failing with different messages, and succeeding in
// between, each see their own.
static void test_threads() {
    std::vector<std::thread> ts;
    for (int i = 0; i < 8; ++i)
        ts.emplace_back([i] {
            hts_desc d = desc(256, 256, 128, 128, HTS_BF16);
            uint8_t map[4] = {0, 1, 1, 0};
            hts_sizes s;
            char want[32];
            std::snprintf(want, sizeof want, "M=-%d ", i + 1);
            for (int r = 0; r < 300; ++r) {
                size_t n = 0;
                EXPECT(hts_gemm_workspace(&d, -(i + 1), &n) == HTS_ERR_SHAPE, "thread %d", i);
                EXPECT(std::strncmp(hts_last_error(), want, std::strlen(want)) == 0, "thread %d sees '%s'", i,
                       hts_last_error());
                EXPECT(hts_pack_plan(&d, map, nullptr, &s) == HTS_OK && hts_last_error()[0] == '\0', "thread %d ok", i);
            }
        });
    for (auto& t : ts) t.join();
}

// A caller mistake the sanitizer must catch inside the library: an index buffer one record
// short, which hts_pack_plan fills past its end.
static int plant_overflow() {
    hts_desc d = desc(512, 512, 128, 128, HTS_BF16);
    uint8_t map[16] = {};
    hts_tile* index = new hts_tile[15];
    hts_sizes s;
    const int st = hts_pack_plan(&d, map, index, &s);
    delete[] index;
    return st == HTS_OK ? 0 : 2;
}

// HTS_DEBUG=1 with host memory standing in for device buffers: every call is refused before any
// launch (the buffers are not device memory), and the debug path itself runs under the sanitizers.
static void test_debug_mode() {
    setenv("HTS_DEBUG", "1", 1);
    const int launches = stub::g.decode + stub::g.prefill + stub::g.pack + stub::g.unpack + stub::g.silu;
    hts_desc d = desc(1024, 512, 128, 128, HTS_BF16);
    const hts_tile* idx = static_cast<const hts_tile*>(dev());
    EXPECT(hts_gemm(&d, idx, dev(), nullptr, 4, dev(), 512, dev(), 1024, HTS_BF16, nullptr, 0, nullptr) ==
               HTS_ERR_INVALID_ARG,
           "debug gemm on host memory");
    EXPECT(std::strstr(hts_last_error(), "not device memory") != nullptr, "debug message");
    EXPECT(hts_pack(&d, idx, dev(), 512, nullptr, dev(4096), nullptr, nullptr) == HTS_ERR_INVALID_ARG, "debug pack");
    EXPECT(hts_unpack(&d, idx, dev(4096), nullptr, dev(), 512, nullptr) == HTS_ERR_INVALID_ARG, "debug unpack");
    EXPECT(hts_dense_gemm(HTS_BF16, 4, 1024, 512, dev(), 512, dev(), 512, dev(), 1024, HTS_F32, nullptr, 0, nullptr) ==
               HTS_ERR_INVALID_ARG,
           "debug dense");
    EXPECT(hts_silu_mul(HTS_BF16, 3, 64, dev(), 64, dev(), 64, dev(), 64, nullptr) == HTS_ERR_INVALID_ARG,
           "debug silu_mul");
    EXPECT(stub::g.decode + stub::g.prefill + stub::g.pack + stub::g.unpack + stub::g.silu == launches,
           "nothing launched in refused debug calls");
    // the allocation-free entry point runs no debug checks
    hts_desc b = desc(11008, 4096, 128, 128, HTS_BF16);
    EXPECT(hts_gemm_noalloc(&b, idx, dev(), nullptr, 1, dev(), 4096, dev(), 11008, HTS_BF16, nullptr) == HTS_OK,
           "noalloc ignores HTS_DEBUG");
    unsetenv("HTS_DEBUG");
}

int main(int argc, char** argv) {
    if (argc > 1 && std::strcmp(argv[1], "--plant-overflow") == 0) return plant_overflow();
    std::mt19937 rng(12345);
    test_plan(rng);
    test_descriptors();
    test_pack_unpack();
    test_gemm();
    test_elementwise_and_wanda();
    test_threads();
    test_debug_mode();
    std::printf("expectations failed: %d, stub checks failed: %d, launches: pack %d masked %d unpack %d streaming %d "
                "tiled %d elementwise %d norms %d cost %d map %d\n",
                fails.load(), stub::g.bad, stub::g.pack, stub::g.pack_masked, stub::g.unpack, stub::g.decode,
                stub::g.prefill, stub::g.silu, stub::g.col_norms, stub::g.wanda_cost, stub::g.wanda_map);
    return (fails.load() == 0 && stub::g.bad == 0) ? 0 : 1;
}
