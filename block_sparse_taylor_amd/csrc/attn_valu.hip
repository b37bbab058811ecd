// Fused PISA forward, plain fp32 VALU version (PISA, §3.4 Algorithm 1
// Phases 1-3; Eqs. 3-5 and 9-10; Piecewise-Taylor-Attention README for the
// gated second-order logit term).
//
// One workgroup of 64 threads per (batch*head, query block); thread t owns
// query row t of the block, its running max m, sum l, tail mass l_tail and
// fp32 accumulator. This is the fp32-input path and the reference GPU path
// for bf16 inputs (values are converted exactly to fp32; no rounding of P).
//   Phase 1: every KV block of S_i (band plus routed ids), keys past T masked.
//   Phase 2: every other block j as one virtual token with logit
//            lam + ln n_j (mass n_j e^lam) and value V-hat_j / n_j.
//   Phase 3: o = (acc + (l_tail / T) (s q) H) / l.
#include <math.h>

#include "common.h"

namespace pisa {
namespace {

constexpr int kRows = 64;

template <typename T, int D>
__global__ __launch_bounds__(kRows) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const double* __restrict__ kbar, const float* __restrict__ vsum, const float* __restrict__ hsum,
    const int32_t* __restrict__ idx, const float* __restrict__ wgate, T* __restrict__ o,
    float* __restrict__ rstat, int Tn,
    int N, float scale, int topk, int band, int n_sink, int second_order, int first_order, int phase_mask) {
    constexpr int kSub = 32;                 // K/V rows staged per step
    __shared__ float sk[kSub * D];
    __shared__ float sv[kSub * D];
    extern __shared__ unsigned char sel[];   // N flags

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int i = blockIdx.x;
    const int r0 = i * kBlock;
    const int rows = min(kBlock, Tn - r0);
    const bool do_exact = phase_mask == 0 || (phase_mask & 1);
    const bool do_virtual = phase_mask == 0 || (phase_mask & 2);
    const bool do_first = (phase_mask == 0 || (phase_mask & 4)) && first_order;
    const int64_t base = bh * (int64_t)Tn * D;
    const int t = r0 + tid;
    const bool active = tid < rows;

    float qv[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qv[d] = active ? load_f32(q + base + (int64_t)t * D + d) * scale : 0.f;  // q' = s q
        acc[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f, ltail = 0.f;

    for (int j = tid; j < N; j += kRows) sel[j] = 0;
    __syncthreads();
    if (tid == 0) {
        for (int j = max(0, i - band); j <= min(N - 1, i + band); ++j) sel[j] = 1;
        for (int j = 0; j < min(n_sink, N); ++j) sel[j] = 1;   // sink blocks
        const int32_t* row = idx ? idx + (bh * (int64_t)N + i) * topk : nullptr;
        for (int c = 0; c < topk; ++c)
            if (row[c] >= 0 && row[c] < N) sel[row[c]] = 1;   // anything else counts as padding
    }
    __syncthreads();

    // Phase 1: exact blocks, ascending j.
    if (do_exact) {
        for (int j = 0; j < N; ++j) {
            if (!sel[j]) continue;
            const int nj = min(kBlock, Tn - j * kBlock);
            for (int h0 = 0; h0 < nj; h0 += kSub) {
            const int nh = min(kSub, nj - h0);
            const int64_t src = base + ((int64_t)j * kBlock + h0) * D;
            __syncthreads();
            for (int c = tid; c < nh * D; c += kRows) {
                sk[c] = load_f32(k + src + c);
                sv[c] = load_f32(v + src + c);
            }
            __syncthreads();
            for (int n = 0; n < nh; ++n) {
                float z = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) z = fmaf(qv[d], sk[n * D + d], z);
                if (z > m) {
                    const float c = expf(m - z);
                    l *= c;
                    ltail *= c;
#pragma unroll
                    for (int d = 0; d < D; ++d) acc[d] *= c;
                    m = z;
                }
                const float p = expf(z - m);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sv[n * D + d], acc[d]);
            }
            }
        }
    }

    // Phase 2: virtual tokens of the unselected blocks, kbar (as fp32) and
    // V-hat of kSub consecutive blocks staged in LDS at a time.
    if (do_virtual) {
        const double* kb = kbar + bh * (int64_t)N * D;
        const float* vs = vsum + bh * (int64_t)N * D;
        const float* wr = second_order ? wgate + (bh * (int64_t)N + i) * N : nullptr;
        for (int j0 = 0; j0 < N; j0 += kSub) {
            const int nh = min(kSub, N - j0);
            __syncthreads();
            for (int c = tid; c < nh * D; c += kRows) {
                sk[c] = (float)kb[(int64_t)j0 * D + c];
                sv[c] = vs[(int64_t)j0 * D + c];
            }
            __syncthreads();
            for (int n = 0; n < nh; ++n) {
                const int j = j0 + n;
                if (sel[j]) continue;
                const int nj = min(kBlock, Tn - j * kBlock);
                float z = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) z = fmaf(qv[d], sk[n * D + d], z);
                if (second_order) z += wr[j];
                const float lnn = logf((float)nj);
                const float zm = z + lnn;
                if (zm > m) {
                    const float c = expf(m - zm);
                    l *= c;
                    ltail *= c;
#pragma unroll
                    for (int d = 0; d < D; ++d) acc[d] *= c;
                    m = zm;
                }
                const float a = expf(z - m);     // e^{lam - m}
                const float mass = a * (float)nj;
                l += mass;
                ltail += mass;
#pragma unroll
                for (int d = 0; d < D; ++d) acc[d] = fmaf(a, sv[n * D + d], acc[d]);
            }
        }
    }

    // Phase 3: global first order, acc += (l_tail / T) (s q) H, with H staged
    // in LDS kSub rows at a time (every thread takes part in the staging).
    if (do_first) {
        const float* H = hsum + bh * (int64_t)D * D;
        const float cf = ltail > 0.f ? ltail / (float)Tn : 0.f;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += kSub) {
            __syncthreads();
            for (int c = tid; c < kSub * D; c += kRows) sk[c] = H[(int64_t)d0 * D + c];
            __syncthreads();
#pragma unroll
            for (int d = 0; d < kSub; ++d) {
                const float w = cf * qv[d0 + d];
#pragma unroll
                for (int e = 0; e < D; ++e) acc[e] = fmaf(w, sk[d * D + e], acc[e]);
            }
        }
    }
    if (active) {
        const float inv = 1.f / l;
#pragma unroll
        for (int d = 0; d < D; ++d) o[base + (int64_t)t * D + d] = store_cast<T>(acc[d] * inv);
        if (rstat != nullptr) {   // the row's lse and c
            const int64_t rr = 2 * (bh * (int64_t)Tn + t);
            rstat[rr] = m + logf(l);
            rstat[rr + 1] = do_first ? ltail / l / (float)Tn : 0.f;
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd_valu(const Geom& g, int dtype, const pisa_params_t* p, const void* q,
                                const void* k, const void* v, const StatsView* st,
                                const int32_t* idx, const float* wgate, void* o, float* rstat,
                                hipStream_t stream) {
    dim3 grid(g.N, (unsigned)g.BH), block(kRows);
    const size_t shm = (size_t)g.N;
#define PISA_VALU_LAUNCH(TT, DD)                                                                   \
    hipLaunchKernelGGL((attn_valu_kernel<TT, DD>), grid, block, shm, stream,                       \
                       static_cast<const TT*>(q), static_cast<const TT*>(k),                       \
                       static_cast<const TT*>(v), st->kbar, st->vsum, st->hsum, idx, wgate,        \
                       static_cast<TT*>(o), rstat, g.T, g.N, g.scale, p->topk, p->band, p->n_sink, p->second_order,  \
                       p->first_order, p->phase_mask)
    if (dtype == PISA_BF16) {
        if (g.D == 128) PISA_VALU_LAUNCH(bf16_t, 128);
        else PISA_VALU_LAUNCH(bf16_t, 64);
    } else {
        if (g.D == 128) PISA_VALU_LAUNCH(float, 128);
        else PISA_VALU_LAUNCH(float, 64);
    }
#undef PISA_VALU_LAUNCH
    return hipGetLastError();
}

}  // namespace pisa
