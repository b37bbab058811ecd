// Covariance-aware routing prior (PISA, §3.3 "Covariance-Aware Block
// Selection", Eq. 11, and Appendix D; Piecewise-Taylor-Attention README:
// cov_bias=True, the router's per-block Frobenius norm):
//
//   M_j = || H_j - Hbar ||_F,  H_j = sum_n (k_{j,n} - kbar_j)^T v_{j,n},
//   Hbar = (1/N) sum_j H_j   (the global statistic of Eq. 10),
//
// and the router adds log(M_j + eps) to block j's pooled score. The routing
// decisions are meant to equal a float64 evaluation, so M_j is formed in fp64
// from the exact inputs (bf16 and fp32 values are exact in fp64): a rounded
// fp32 H_j or Hbar would move log M_j by far more than the score gaps the
// router settles. Two passes over K and V, only when the prior is asked for:
//   1. cov_partial_kernel: per (head, range of blocks) the fp64 sum of the
//      range's H_j; cov_reduce_kernel adds the ranges of a head in a fixed
//      order and divides by N (Hbar, fp64).
//   2. cov_norm_kernel: per block, H_j - Hbar in fp64 and its Frobenius norm.
// Each thread of a workgroup owns a (D/16) x (D/16) tile of the D x D matrix
// in fp64 registers; a block's K and V rows are staged in LDS as fp32 (exact)
// and every row contributes one rank-1 update of the tile: a dense fp64
// contraction over the block's 64 rows, on the fp64 FMA units.
#include <algorithm>

#include "common.h"

namespace pisa {
namespace {

template <typename T> __device__ __forceinline__ float4 load4(const T* p);
template <> __device__ __forceinline__ float4 load4<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

// Accumulate H_j = sum_n (k_n - kbar_j)^T v_n of block j into this thread's
// tile acc[TD][TD] (rows a0 .., columns b0 ..), staging the block's rows in
// LDS (fp32, row pitch D + 4). Rows past T are zero in V, so they add nothing.
template <typename T, int D>
__device__ __forceinline__ void block_product(const T* __restrict__ k, const T* __restrict__ v,
                                              const double* __restrict__ kbar, int64_t bh, int T_, int N,
                                              int j, float* ks, float* vs, double* kb_s,
                                              double (&acc)[D / 16][D / 16], int a0, int b0) {
    constexpr int TD = D / 16;
    constexpr int LD = D + 4;
    const int tid = threadIdx.x;
    const int rows = min(kBlock, T_ - j * kBlock);
    const T* kh = k + (bh * (int64_t)T_ + (int64_t)j * kBlock) * D;
    const T* vh = v + (bh * (int64_t)T_ + (int64_t)j * kBlock) * D;
    __syncthreads();   // the previous block's LDS reads are done
    for (int c = tid; c < kBlock * (D / 4); c += kThreads) {
        const int r = c / (D / 4), d4 = c % (D / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
        if (r < rows) {
            x = load4<T>(kh + (int64_t)r * D + 4 * d4);
            y = load4<T>(vh + (int64_t)r * D + 4 * d4);
        }
        *reinterpret_cast<float4*>(ks + r * LD + 4 * d4) = x;
        *reinterpret_cast<float4*>(vs + r * LD + 4 * d4) = y;
    }
    if (tid < D) kb_s[tid] = kbar[(bh * N + j) * (int64_t)D + tid];
    __syncthreads();
    double kbt[TD];
#pragma unroll
    for (int x = 0; x < TD; ++x) kbt[x] = kb_s[a0 + x];
    for (int r = 0; r < kBlock; ++r) {
        double dk[TD], vv[TD];
#pragma unroll
        for (int x4 = 0; x4 < TD / 4; ++x4) {
            const float4 a = *reinterpret_cast<const float4*>(ks + r * LD + a0 + 4 * x4);
            const float4 b = *reinterpret_cast<const float4*>(vs + r * LD + b0 + 4 * x4);
            dk[4 * x4 + 0] = (double)a.x - kbt[4 * x4 + 0];
            dk[4 * x4 + 1] = (double)a.y - kbt[4 * x4 + 1];
            dk[4 * x4 + 2] = (double)a.z - kbt[4 * x4 + 2];
            dk[4 * x4 + 3] = (double)a.w - kbt[4 * x4 + 3];
            vv[4 * x4 + 0] = (double)b.x;
            vv[4 * x4 + 1] = (double)b.y;
            vv[4 * x4 + 2] = (double)b.z;
            vv[4 * x4 + 3] = (double)b.w;
        }
#pragma unroll
        for (int x = 0; x < TD; ++x)
#pragma unroll
            for (int y = 0; y < TD; ++y) acc[x][y] = fma(dk[x], vv[y], acc[x][y]);
    }
}

// Pass 1: workgroup (g, bh) sums H_j over blocks [g bpr, min(N, g bpr + bpr)).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void cov_partial_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                               const double* __restrict__ kbar, int T_, int N,
                                                               int bpr, double* __restrict__ part) {
    constexpr int TD = D / 16;
    __shared__ __attribute__((aligned(16))) float ks[kBlock * (D + 4)];
    __shared__ __attribute__((aligned(16))) float vs[kBlock * (D + 4)];
    __shared__ double kb_s[D];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int a0 = (tid / 16) * TD, b0 = (tid % 16) * TD;
    double acc[TD][TD];
#pragma unroll
    for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) acc[x][y] = 0.0;
    const int j1 = min(N, (g + 1) * bpr);
    for (int j = g * bpr; j < j1; ++j) block_product<T, D>(k, v, kbar, bh, T_, N, j, ks, vs, kb_s, acc, a0, b0);
    double* out = part + (bh * gridDim.x + g) * (int64_t)D * D;
#pragma unroll
    for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) out[(a0 + x) * D + b0 + y] = acc[x][y];
}

// Hbar of each head: the ranges' partial sums in a fixed order, over N.
__global__ __launch_bounds__(kThreads) void cov_reduce_kernel(const double* __restrict__ part, int G, int D, int N,
                                                              double* __restrict__ hbar) {
    const int64_t bh = blockIdx.y;
    const int DD = D * D;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= DD) return;
    const double* p = part + bh * (int64_t)G * DD + e;
    double s = 0.0;
    for (int g = 0; g < G; ++g) s += p[(int64_t)g * DD];
    hbar[bh * DD + e] = s / (double)N;
}

// Pass 2: workgroup (j, bh) forms H_j - Hbar and writes M_j = its Frobenius norm.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void cov_norm_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                            const double* __restrict__ kbar, int T_, int N,
                                                            const double* __restrict__ hbar,
                                                            double* __restrict__ hnorm) {
    constexpr int TD = D / 16;
    __shared__ __attribute__((aligned(16))) float ks[kBlock * (D + 4)];
    __shared__ __attribute__((aligned(16))) float vs[kBlock * (D + 4)];
    __shared__ double kb_s[D];
    __shared__ double red[kThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t bh = blockIdx.y;
    const int j = blockIdx.x;
    const int a0 = (tid / 16) * TD, b0 = (tid % 16) * TD;
    double acc[TD][TD];
    const double* hb = hbar + bh * (int64_t)D * D;
#pragma unroll
    for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) acc[x][y] = -hb[(a0 + x) * D + b0 + y];
    block_product<T, D>(k, v, kbar, bh, T_, N, j, ks, vs, kb_s, acc, a0, b0);
    double ss = 0.0;
#pragma unroll
    for (int x = 0; x < TD; ++x)
#pragma unroll
        for (int y = 0; y < TD; ++y) ss = fma(acc[x][y], acc[x][y], ss);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if (lane == 0) red[tid >> 6] = ss;
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
        for (int w = 0; w < kThreads / 64; ++w) t += red[w];
        hnorm[bh * N + j] = sqrt(t);
    }
}

// Ranges per head of pass 1: the fp64 partials plus Hbar fit in the bytes the
// statistics pass's fp32 partials take (half as many ranges, less one), and
// at least one.
int cov_ranges(const Geom& g, int stats_groups) { return std::max(1, std::min(g.N, stats_groups / 2 - 1)); }

}  // namespace

size_t cov_workspace_bytes(const Geom& g, int stats_groups) {
    return (size_t)g.BH * (cov_ranges(g, stats_groups) + 1) * g.D * g.D * sizeof(double);
}

hipError_t launch_cov_norm(const Geom& g, int dtype, const void* k, const void* v, const double* kbar,
                           double* hnorm, void* workspace, int stats_groups, hipStream_t stream) {
    const int G = cov_ranges(g, stats_groups);
    const int bpr = (g.N + G - 1) / G;
    const int Gu = (g.N + bpr - 1) / bpr;   // ranges actually used
    double* part = static_cast<double*>(workspace);
    double* hbar = part + (size_t)g.BH * Gu * g.D * g.D;
    const dim3 block(kThreads);
#define PISA_COV_LAUNCH(TT, DD)                                                                           \
    do {                                                                                                  \
        hipLaunchKernelGGL((cov_partial_kernel<TT, DD>), dim3(Gu, (unsigned)g.BH), block, 0, stream,     \
                           static_cast<const TT*>(k), static_cast<const TT*>(v), kbar, g.T, g.N, bpr, part); \
        hipLaunchKernelGGL(cov_reduce_kernel, dim3((DD * DD + kThreads - 1) / kThreads, (unsigned)g.BH),  \
                           block, 0, stream, part, Gu, DD, g.N, hbar);                                    \
        hipLaunchKernelGGL((cov_norm_kernel<TT, DD>), dim3(g.N, (unsigned)g.BH), block, 0, stream,       \
                           static_cast<const TT*>(k), static_cast<const TT*>(v), kbar, g.T, g.N, hbar,   \
                           hnorm);                                                                        \
    } while (0)
    if (dtype == PISA_BF16) {
        if (g.D == 128) PISA_COV_LAUNCH(bf16_t, 128);
        else PISA_COV_LAUNCH(bf16_t, 64);
    } else {
        if (g.D == 128) PISA_COV_LAUNCH(float, 128);
        else PISA_COV_LAUNCH(float, 64);
    }
#undef PISA_COV_LAUNCH
    return hipGetLastError();
}

}  // namespace pisa
