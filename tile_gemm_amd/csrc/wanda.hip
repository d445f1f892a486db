// Wanda-derived tile maps on gfx950 (page "SparseGPT vs Wanda: one-shot LLM
// pruning without retraining", Wanda section: a weight's importance is its
// magnitude times the input activation of its column; the lowest are removed).
// Column scale = L2 norm of the calibration activations of each column; a
// tile's cost = the score mass a 2:4 mask of it would drop; the layer keeps its
// costliest tiles dense and makes the n_sparse cheapest ones 2:4 (page "PATCH:
// Learnable Tile-level Hybrid Sparsity for LLMs", section 2: a per-tile dense /
// 2:4 choice; learning that choice is not done here, the map is derived).
#include "device_common.h"
#include "hts_internal.h"

namespace hts {
namespace {

// Correctly rounded binary32 square root of a non-negative binary64 value:
// start from the conversion of the binary64 root, then settle the rounding by
// comparing s with the exact square of the midpoint between neighbours (a float
// has 24 bits, so squares of floats and of their midpoints are exact in binary64).
__device__ float sqrt_to_f32(double s) {
    float r = (float)sqrt(s);
    for (int it = 0; it < 2; ++it) {
        const float up = nextafterf(r, INFINITY), dn = nextafterf(r, 0.f);
        const double mu = 0.5 * ((double)r + (double)up), md = 0.5 * ((double)r + (double)dn);
        if (s > mu * mu || (s == mu * mu && (__float_as_uint(up) & 1u) == 0u)) r = up;
        else if (s < md * md || (s == md * md && (__float_as_uint(dn) & 1u) == 0u && r > 0.f)) r = dn;
        else break;
    }
    return r;
}

template <typename T>
__global__ __launch_bounds__(256) void col_norms_kernel(int64_t rows, int64_t K, const uint16_t* __restrict__ X,
                                                        int64_t ldx, float* __restrict__ out) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    double acc = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        const double x = (double)widen<T>(X[r * ldx + k]);
        const double sq = x * x;                       // exact: a 16-bit value squared
        acc = acc + sq;
    }
    out[k] = sqrt_to_f32(acc);
}

__device__ __forceinline__ void keep_rule(const float s[4], bool keep[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int rank = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j == i) continue;
            rank += (s[j] > s[i]) || (s[j] == s[i] && j < i);
        }
        keep[i] = rank < 2;
    }
}

// One workgroup per tile, one thread per tile row; row sums in group order, then
// row sums added in row order by thread 0.
template <typename T>
__global__ __launch_bounds__(128) void wanda_cost_kernel(int64_t Tk, int bn, int bk, const uint16_t* __restrict__ W,
                                                         int64_t ldw, const float* __restrict__ cs,
                                                         double* __restrict__ cost) {
    __shared__ double rowsum[128];
    const int64_t t = blockIdx.x, tn = t / Tk, tk = t % Tk;
    const int r = threadIdx.x;
    if (r < bn) {
        const uint16_t* src = W + (tn * bn + r) * ldw + tk * bk;
        const float* c = cs + tk * bk;
        double acc = 0.0;
        for (int g = 0; g < bk / 4; ++g) {
            const uint2 q = *reinterpret_cast<const uint2*>(src + 4 * g);
            const uint32_t b[4] = {q.x & 0xFFFFu, q.x >> 16, q.y & 0xFFFFu, q.y >> 16};
            float s[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) s[i] = fabsf(widen<T>(b[i])) * c[4 * g + i];
            bool keep[4];
            keep_rule(s, keep);
            // the two dropped scores, lower index first
            const float lo = !keep[0] ? s[0] : (!keep[1] ? s[1] : s[2]);
            const float hi = !keep[3] ? s[3] : (!keep[2] ? s[2] : s[1]);
            acc = acc + ((double)lo + (double)hi);
        }
        rowsum[r] = acc;
    }
    __syncthreads();
    if (r == 0) {
        double total = 0.0;
        for (int i = 0; i < bn; ++i) total = total + rowsum[i];
        cost[t] = total;
    }
}

__global__ __launch_bounds__(256) void wanda_map_kernel(int64_t T, const double* __restrict__ cost, int64_t n_sparse,
                                                        uint8_t* __restrict__ map) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const double ct = cost[t];
    int64_t rank = 0;
    for (int64_t u = 0; u < T; ++u) {
        const double cu = cost[u];
        rank += (cu < ct) || (cu == ct && u < t);
    }
    map[t] = rank < n_sparse ? (uint8_t)HTS_TILE_SPARSE24 : (uint8_t)HTS_TILE_DENSE;
}

}  // namespace

hipError_t launch_col_norms(int32_t dtype, int64_t rows, int64_t K, const uint16_t* X, int64_t ldx, float* out,
                            hipStream_t s) {
    const dim3 grid((unsigned)((K + 255) / 256));
    if (dtype == HTS_BF16)
        col_norms_kernel<BF16T><<<grid, dim3(256), 0, s>>>(rows, K, X, ldx, out);
    else
        col_norms_kernel<F16T><<<grid, dim3(256), 0, s>>>(rows, K, X, ldx, out);
    return hipGetLastError();
}

hipError_t launch_wanda_cost(const hts_desc& d, const uint16_t* W, int64_t ldw, const float* cs, double* cost,
                             hipStream_t s) {
    const int64_t Tk = d.K / d.bk, T = (d.N / d.bn) * Tk;
    if (d.dtype == HTS_BF16)
        wanda_cost_kernel<BF16T><<<dim3((unsigned)T), dim3(128), 0, s>>>(Tk, d.bn, d.bk, W, ldw, cs, cost);
    else
        wanda_cost_kernel<F16T><<<dim3((unsigned)T), dim3(128), 0, s>>>(Tk, d.bn, d.bk, W, ldw, cs, cost);
    return hipGetLastError();
}

hipError_t launch_wanda_map(int64_t T, const double* cost, int64_t n_sparse, uint8_t* map, hipStream_t s) {
    wanda_map_kernel<<<dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s>>>(T, cost, n_sparse, map);
    return hipGetLastError();
}

}  // namespace hts
