// Elementwise step of a gated MLP between hybrid products: H = silu(G) * U, silu(x) = x / (1 + e^-x).
//
// In a LLaMA-style decoder block the gate and up projections both read the block input and the
// down projection reads silu(gate) * up; this kernel is that step, so the seven projections of a
// block can run back to back on packed weights.  HBM-bound: reads G and U, writes H, once each.
// Each thread handles 8 consecutive elements with 16-byte loads and stores (fp32 arithmetic,
// one rounding to the 16-bit type).
#include "device_common.h"
#include "hts_internal.h"

namespace hts {
namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(int64_t M, int64_t N, const uint16_t* __restrict__ G,
                                                            int64_t ldg, const uint16_t* __restrict__ U, int64_t ldu,
                                                            uint16_t* __restrict__ H, int64_t ldh) {
    const int64_t per_row = N / 8, total = M * per_row;
    for (int64_t it = (int64_t)blockIdx.x * kThreads + threadIdx.x; it < total;
         it += (int64_t)gridDim.x * kThreads) {
        const int64_t m = it / per_row, c = (it - m * per_row) * 8;
        const u32x4 g = ld16(G + m * ldg + c), u = ld16(U + m * ldu + c);
        u32x4 h;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t out = 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const float x = widen<T>((g[w] >> (16 * half)) & 0xFFFFu);
                const float y = widen<T>((u[w] >> (16 * half)) & 0xFFFFu);
                const float v = x / (1.0f + expf(-x)) * y;
                const uint32_t b = (T::id == BF16T::id) ? narrow_bf16(v) : narrow_f16(v);
                out |= b << (16 * half);
            }
            h[w] = out;
        }
        st16(H + m * ldh + c, h);
    }
}

}  // namespace

hipError_t launch_silu_mul(int32_t dtype, int64_t M, int64_t N, const uint16_t* G, int64_t ldg, const uint16_t* U,
                           int64_t ldu, uint16_t* H, int64_t ldh, hipStream_t s) {
    const int64_t work = M * (N / 8);
    const int64_t blocks64 = (work + kThreads - 1) / kThreads;
    const unsigned blocks = (unsigned)(blocks64 < 8192 ? blocks64 : 8192);
    if (dtype == HTS_BF16)
        silu_mul_kernel<BF16T><<<dim3(blocks), dim3(kThreads), 0, s>>>(M, N, G, ldg, U, ldu, H, ldh);
    else
        silu_mul_kernel<F16T><<<dim3(blocks), dim3(kThreads), 0, s>>>(M, N, G, ldg, U, ldu, H, ldh);
    return hipGetLastError();
}

}  // namespace hts
