// What the launcher stand-ins record (host-only sanitizer build of the C API).
#pragma once
#include <cstddef>
#include <cstdint>

namespace stub {
struct Log {
    int pack = 0, pack_masked = 0, unpack = 0, decode = 0, prefill = 0, silu = 0, col_norms = 0;
    int wanda_cost = 0, wanda_map = 0;
    int bad = 0;                 // failed checks
    int last_nsplit = 0;
    const void* ws = nullptr;    // the workspace the driver passed (bounds for the checks)
    size_t ws_bytes = 0;
    bool expect_unpack_ws = false;
};
extern Log g;
void complain(const char* what);
}  // namespace stub
