// Pooled-score routing (PISA, Algorithm 1 step 2 with the pooled block score
// of Eq. 11 minus its covariance term; Piecewise-Taylor-Attention README:
// +-band forced exact, clamped ranking spread min(w, ln B), set-identical
// top-k).
//
// One workgroup per (batch*head, tile of query blocks). For each query block:
//   1. pool its rows: qbar = mean(q), q2bar = mean((s q)^2)        (fp64, exact sums)
//   2. score every KV block j: r_j = s qbar.kbar_j [+ min(w_j, ln B)], with
//      w_j = 1/2 q2bar.ksig2_j; the band |i-j| <= band is excluded   (fp64)
//   3. radix-select the topk-th largest 64-bit order-preserving key, then
//      keep every key above it plus the lowest-index keys equal to it
//   4. write the chosen ids ascending (block prefix sum), then -1 padding.
// The score row lives only in LDS; nothing N x N is written except the
// gated second-order table the fused kernel consumes.
#include <math.h>

#include "common.h"

namespace pisa {
namespace {

constexpr int kMaxN = 8192;   // LDS-resident key row (64 KiB)

__device__ __forceinline__ uint64_t order_key(double r) {
    r = r + 0.0;  // -0 -> +0
    uint64_t u = __double_as_longlong(r);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Block-wide exclusive prefix sum over kThreads ints; returns the total.
__device__ __forceinline__ int block_scan(int x, int* scratch, int* excl) {
    const int tid = threadIdx.x;
    scratch[tid] = x;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        int y = tid >= off ? scratch[tid - off] : 0;
        __syncthreads();
        scratch[tid] += y;
        __syncthreads();
    }
    const int incl = scratch[tid];
    const int total = scratch[kThreads - 1];
    __syncthreads();
    *excl = incl - x;
    return total;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const T* __restrict__ q, const double* __restrict__ kbar, const double* __restrict__ ksig2,
    int Tn, int N, float scale, int topk, int band, int second_order, int32_t* __restrict__ idx,
    float* __restrict__ wgate) {
    __shared__ double qbar_s[D];
    __shared__ double q2_s[D];
    __shared__ uint64_t key_s[kMaxN];
    __shared__ unsigned hist[256];
    __shared__ int scan_s[kThreads];
    __shared__ uint64_t prefix_s;
    __shared__ int need_s;

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int i = blockIdx.x;
    const T* qh = q + bh * (int64_t)Tn * D;
    const int r0 = i * kBlock;
    const int rows = min(kBlock, Tn - r0);
    const double s = (double)scale;
    const double lnB = log((double)kBlock);

    // 1. pooling
    if (tid < D) {
        double a = 0.0, b = 0.0;
        for (int n = 0; n < rows; ++n) {
            const double x = (double)load_f32(qh + (int64_t)(r0 + n) * D + tid);
            a += x;
            const double y = s * x;
            b += y * y;
        }
        qbar_s[tid] = a / rows;
        q2_s[tid] = b / rows;
    }
    __syncthreads();

    // 2. scores (candidates only; band entries get key 0, below every real key)
    const double* kb = kbar + bh * (int64_t)N * D;
    const double* sg = second_order ? ksig2 + bh * (int64_t)N * D : nullptr;
    float* wrow = second_order ? wgate + (bh * (int64_t)N + i) * N : nullptr;
    int ncand = 0;
    for (int j = tid; j < N; j += kThreads) {
        double dot = 0.0;
        const double* kr = kb + (int64_t)j * D;
        for (int d = 0; d < D; ++d) dot = fma(qbar_s[d], kr[d], dot);
        double r = s * dot;
        if (second_order) {
            const double* sr = sg + (int64_t)j * D;
            double w = 0.0;
            for (int d = 0; d < D; ++d) w = fma(q2_s[d], sr[d], w);
            w *= 0.5;
            r += fmin(w, lnB);
            wrow[j] = (float)(w > lnB ? 0.0 : w);
        }
        const bool cand = abs(i - j) > band;
        key_s[j] = cand ? order_key(r) : 0ull;
        ncand += cand;
    }
    // count candidates
    int dummy;
    ncand = block_scan(ncand, scan_s, &dummy);
    const int k = min(topk, ncand);
    int32_t* out = idx + (bh * (int64_t)N + i) * topk;
    if (k == 0) {
        for (int c = tid; c < topk; c += kThreads) out[c] = -1;
        return;
    }

    // 3. radix select of the k-th largest key (8 passes of 8 bits, MSB first)
    if (tid == 0) { prefix_s = 0ull; need_s = k; }
    __syncthreads();
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        const uint64_t hmask = pass == 0 ? 0ull : (~0ull << (shift + 8));
        hist[tid] = 0;
        __syncthreads();
        const uint64_t pre = prefix_s;
        for (int j = tid; j < N; j += kThreads) {
            const uint64_t key = key_s[j];
            if (key != 0ull && (key & hmask) == pre) atomicAdd(&hist[(key >> shift) & 255], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            int need = need_s;
            int digit = 255;
            for (; digit > 0; --digit) {
                const int c = (int)hist[digit];
                if (c >= need) break;
                need -= c;
            }
            prefix_s = pre | ((uint64_t)digit << shift);
            need_s = need;
        }
        __syncthreads();
    }
    const uint64_t thr = prefix_s;   // the k-th largest key
    const int need_eq = need_s;       // how many keys equal to thr are taken (lowest index first)

    // 4. chosen = key > thr, or key == thr among the first need_eq such keys in j order.
    // Pass A: rank the equal keys in j order; pass B: write ids ascending.
    int written = 0, eq_seen = 0;
    for (int base = 0; base < N; base += kThreads) {
        const int j = base + tid;
        const uint64_t key = j < N ? key_s[j] : 0ull;
        const int is_eq = (key == thr && key != 0ull) ? 1 : 0;
        int eq_before;
        const int eq_tot = block_scan(is_eq, scan_s, &eq_before);
        const int take = (key > thr) || (is_eq && (eq_seen + eq_before) < need_eq);
        int pos;
        const int tot = block_scan(take, scan_s, &pos);
        if (take && written + pos < topk) out[written + pos] = j;
        written += tot;
        eq_seen += eq_tot;
    }
    for (int c = written + tid; c < topk; c += kThreads) out[c] = -1;
}

}  // namespace

hipError_t launch_route_topk(const Geom& g, int dtype, const pisa_params_t* p, const void* q,
                             const pisa_stats_t* st, int32_t* idx, float* wgate, hipStream_t stream) {
    dim3 grid(g.N, (unsigned)g.BH), block(kThreads);
    const int so = p->second_order;
    if (p->topk == 0 && !so) return hipSuccess;
    int32_t* out = idx;
    // topk == 0 with the second-order table requested: still run for wgate.
    if (dtype == PISA_BF16) {
        auto qq = static_cast<const bf16_t*>(q);
        if (g.D == 128)
            hipLaunchKernelGGL((route_kernel<bf16_t, 128>), grid, block, 0, stream, qq, st->kbar,
                               st->ksig2, g.T, g.N, g.scale, p->topk, p->band, so, out, wgate);
        else
            hipLaunchKernelGGL((route_kernel<bf16_t, 64>), grid, block, 0, stream, qq, st->kbar,
                               st->ksig2, g.T, g.N, g.scale, p->topk, p->band, so, out, wgate);
    } else {
        auto qq = static_cast<const float*>(q);
        if (g.D == 128)
            hipLaunchKernelGGL((route_kernel<float, 128>), grid, block, 0, stream, qq, st->kbar,
                               st->ksig2, g.T, g.N, g.scale, p->topk, p->band, so, out, wgate);
        else
            hipLaunchKernelGGL((route_kernel<float, 64>), grid, block, 0, stream, qq, st->kbar,
                               st->ksig2, g.T, g.N, g.scale, p->topk, p->band, so, out, wgate);
    }
    return hipGetLastError();
}

}  // namespace pisa
