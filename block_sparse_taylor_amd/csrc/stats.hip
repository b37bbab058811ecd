// Block statistics of K and V (PISA, Algorithm 1 step 1 / Fig. 4 "Prepare
// Phase"; Appendix C notation; Piecewise-Taylor-Attention README, "Blog
// post" for the per-dimension key variance and the changelog's "hc-free"
// identity sum_j (K_j - kbar_j)^T V_j = K^T V - sum_j kbar_j (x) V-hat_j).
//
// One workgroup streams BPW consecutive 64-row blocks of one (batch, head):
//   * column statistics per block (kbar, V-hat, sigma^2) in fp64 from the
//     exact input values, written once per block;
//   * the partial first-order matrix sum_j (K_j^T V_j - kbar_j (x) V-hat_j)
//     accumulated on chip: bf16 inputs use bf16 MFMA (exact products, fp32
//     accumulation), fp32 inputs an fp64 VALU loop;
//   * the partial is written to the workspace, and a second kernel adds the
//     partials of a head in a fixed order (no atomics, deterministic).
// HBM traffic: K and V are read once (2 B T D bytes per head in bf16).
#include "common.h"

namespace pisa {
namespace {

constexpr int kPad = 4;  // LDS row padding (elements): rows 8 apart fall on disjoint bank halves

template <int D> constexpr int bpw() { return 32; }

// ---------------------------------------------------------------- column statistics
template <typename T, int D>
__device__ __forceinline__ void column_stats(const T* tile_k, const T* tile_v, int ld, int rows,
                                             int64_t out_off, int second_order, double* kbar,
                                             float* vsum, double* ksig2, T* kbar_c, T* vbar_c,
                                             float* kb_s, float* vs_s) {
    const int tid = threadIdx.x;
    if (tid < D) {
        const int d = tid;
        double s = 0.0;
        for (int n = 0; n < rows; ++n) s += (double)load_f32(tile_k + n * ld + d);
        const double mean = s / (double)rows;
        kbar[out_off + d] = mean;
        kbar_c[out_off + d] = store_cast<T>((float)mean);
        kb_s[d] = (float)mean;
        if (second_order) {
            double q = 0.0;
            for (int n = 0; n < rows; ++n) {
                const double x = (double)load_f32(tile_k + n * ld + d) - mean;
                q += x * x;
            }
            ksig2[out_off + d] = q / (double)rows;
        }
    } else if (tid < 2 * D) {
        const int d = tid - D;
        double s = 0.0;
        for (int n = 0; n < rows; ++n) s += (double)load_f32(tile_v + n * ld + d);
        vsum[out_off + d] = (float)s;
        vbar_c[out_off + d] = store_cast<T>((float)(s / (double)rows));
        vs_s[d] = (float)s;
    }
}

// ---------------------------------------------------------------- bf16 path (MFMA)
// 32x32x16 bf16 MFMA operand layout (lane l, element e in 0..7):
//   A[m = l%32][k = 8(l/32) + e],  B[k = 8(l/32) + e][n = l%32]
//   C[m = 8(i/4) + 4(l/32) + i%4][n = l%32] for accumulator register i.
// H^T-free form: C[a][b] += sum_t K[t][a] V[t][b], so A = K^T and B = V, both
// gathered column-wise from the row-major LDS tiles.
template <int D>
__global__ __launch_bounds__(kThreads) void stats_bf16_kernel(
    const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, int T, int N, int second_order,
    double* __restrict__ kbar, float* __restrict__ vsum, double* __restrict__ ksig2,
    bf16_t* __restrict__ kbar_c, bf16_t* __restrict__ vbar_c, float* __restrict__ hpart) {
    constexpr int BPW = bpw<D>();
    constexpr int LD = D + kPad;
    constexpr int CH = D / 8;                       // 16-byte chunks per row
    constexpr int LOADS = kBlock * CH / kThreads;   // uint4 loads per thread per tensor
    constexpr int NT = D / 32;                      // 32-wide tiles per dim
    constexpr int TPW = NT * NT / 4;                // output tiles per wave
    __shared__ __attribute__((aligned(16))) bf16_t sk[kBlock * LD];
    __shared__ __attribute__((aligned(16))) bf16_t sv[kBlock * LD];
    __shared__ float kb_s[D];
    __shared__ float vs_s[D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int j0 = g * BPW;
    const int j1 = min(N, j0 + BPW);
    const bf16_t* kh = k + bh * (int64_t)T * D;
    const bf16_t* vh = v + bh * (int64_t)T * D;

    f32x16_t acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

    uint4 pk[LOADS], pv[LOADS];
    auto fetch = [&](int j) {
        const int r0 = j * kBlock;
#pragma unroll
        for (int L = 0; L < LOADS; ++L) {
            const int c = L * kThreads + tid;
            const int row = c / CH, ch = c % CH;
            const int t = r0 + row;
            if (t < T) {
                pk[L] = *reinterpret_cast<const uint4*>(kh + (int64_t)t * D + ch * 8);
                pv[L] = *reinterpret_cast<const uint4*>(vh + (int64_t)t * D + ch * 8);
            } else {
                pk[L] = make_uint4(0, 0, 0, 0);
                pv[L] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    fetch(j0);

    for (int j = j0; j < j1; ++j) {
        const int rows = min(kBlock, T - j * kBlock);
        __syncthreads();  // previous block's LDS reads are done
#pragma unroll
        for (int L = 0; L < LOADS; ++L) {
            const int c = L * kThreads + tid;
            const int row = c / CH, ch = c % CH;
            uint2* dk = reinterpret_cast<uint2*>(sk + row * LD + ch * 8);
            uint2* dv = reinterpret_cast<uint2*>(sv + row * LD + ch * 8);
            dk[0] = make_uint2(pk[L].x, pk[L].y);
            dk[1] = make_uint2(pk[L].z, pk[L].w);
            dv[0] = make_uint2(pv[L].x, pv[L].y);
            dv[1] = make_uint2(pv[L].z, pv[L].w);
        }
        __syncthreads();
        if (j + 1 < j1) fetch(j + 1);

        const int64_t off = (bh * N + j) * D;
        column_stats<bf16_t, D>(sk, sv, LD, rows, off, second_order, kbar, vsum, ksig2, kbar_c,
                                vbar_c, kb_s, vs_s);

        // acc += K_j^T V_j  (rows >= `rows` are zero in LDS)
        const int m = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < kBlock / 16; ++ks) {
            const int t0 = ks * 16 + hi * 8;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int tile = wave * TPW + t;
                const int mt = tile / NT, nt = tile % NT;
                bf16x8_t a, b;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    a[e] = __builtin_bit_cast(__bf16, sk[(t0 + e) * LD + mt * 32 + m]);
                    b[e] = __builtin_bit_cast(__bf16, sv[(t0 + e) * LD + nt * 32 + m]);
                }
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();  // kb_s / vs_s visible
        // acc -= kbar_j (x) V-hat_j
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int tile = wave * TPW + t;
            const int mt = tile / NT, nt = tile % NT;
            const float vb = vs_s[nt * 32 + m];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int a = mt * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
                acc[t][i] -= kb_s[a] * vb;
            }
        }
    }

    float* hp = hpart + ((bh * gridDim.x) + g) * (int64_t)D * D;
    const int m = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile = wave * TPW + t;
        const int mt = tile / NT, nt = tile % NT;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int a = mt * 32 + 8 * (i / 4) + 4 * hi + (i % 4);
            hp[a * D + nt * 32 + m] = acc[t][i];
        }
    }
}

// ---------------------------------------------------------------- fp32 path (VALU, fp64 accumulate)
template <int D>
__global__ __launch_bounds__(kThreads) void stats_f32_kernel(
    const float* __restrict__ k, const float* __restrict__ v, int T, int N, int second_order,
    double* __restrict__ kbar, float* __restrict__ vsum, double* __restrict__ ksig2,
    float* __restrict__ kbar_c, float* __restrict__ vbar_c, float* __restrict__ hpart) {
    constexpr int BPW = bpw<D>();
    constexpr int LD = D + 1;
    constexpr int PER = D * D / kThreads;
    __shared__ float sk[kBlock * LD];
    __shared__ float sv[kBlock * LD];
    __shared__ float kb_s[D];
    __shared__ float vs_s[D];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int j0 = g * BPW, j1 = min(N, j0 + BPW);
    const float* kh = k + bh * (int64_t)T * D;
    const float* vh = v + bh * (int64_t)T * D;
    double acc[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) acc[r] = 0.0;
    for (int j = j0; j < j1; ++j) {
        const int rows = min(kBlock, T - j * kBlock);
        __syncthreads();
        for (int c = tid; c < kBlock * D; c += kThreads) {
            const int row = c / D, col = c % D;
            const int t = j * kBlock + row;
            sk[row * LD + col] = t < T ? kh[(int64_t)t * D + col] : 0.f;
            sv[row * LD + col] = t < T ? vh[(int64_t)t * D + col] : 0.f;
        }
        __syncthreads();
        const int64_t off = (bh * N + j) * D;
        column_stats<float, D>(sk, sv, LD, rows, off, second_order, kbar, vsum, ksig2, kbar_c,
                               vbar_c, kb_s, vs_s);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = tid + r * kThreads;
            const int a = e / D, b = e % D;
            double s = 0.0;
            for (int n = 0; n < rows; ++n) s += (double)sk[n * LD + a] * (double)sv[n * LD + b];
            // kbar (x) V-hat in fp64 from the exact column sums
            double ka = 0.0, vb = 0.0;
            for (int n = 0; n < rows; ++n) {
                ka += (double)sk[n * LD + a];
                vb += (double)sv[n * LD + b];
            }
            acc[r] += s - ka * vb / (double)rows;
        }
    }
    float* hp = hpart + ((bh * gridDim.x) + g) * (int64_t)D * D;
#pragma unroll
    for (int r = 0; r < PER; ++r) hp[tid + r * kThreads] = (float)acc[r];
}

// Fixed-order sum of the per-workgroup partials of each head.
__global__ __launch_bounds__(kThreads) void hsum_reduce_kernel(const float* __restrict__ hpart,
                                                               int G, int DD, float* __restrict__ hsum) {
    const int64_t bh = blockIdx.y;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= DD) return;
    const float* p = hpart + bh * (int64_t)G * DD + e;
    double s = 0.0;
    for (int g = 0; g < G; ++g) s += (double)p[(int64_t)g * DD];
    hsum[bh * DD + e] = (float)s;
}

int stats_groups(const Geom& g) { return (g.N + 31) / 32; }

}  // namespace

size_t stats_workspace_bytes(const Geom& g) {
    return (size_t)g.BH * stats_groups(g) * g.D * g.D * sizeof(float);
}

hipError_t launch_block_stats(const Geom& g, int dtype, int second_order, const void* k, const void* v,
                              const pisa_stats_t* out, void* workspace, hipStream_t stream) {
    const int G = stats_groups(g);
    dim3 grid(G, (unsigned)g.BH), block(kThreads);
    float* hpart = static_cast<float*>(workspace);
    if (dtype == PISA_BF16) {
        auto kc = static_cast<bf16_t*>(out->kbar_c);
        auto vc = static_cast<bf16_t*>(out->vbar_c);
        auto kk = static_cast<const bf16_t*>(k);
        auto vv = static_cast<const bf16_t*>(v);
        if (g.D == 128)
            hipLaunchKernelGGL(stats_bf16_kernel<128>, grid, block, 0, stream, kk, vv, g.T, g.N,
                               second_order, out->kbar, out->vsum, out->ksig2, kc, vc, hpart);
        else
            hipLaunchKernelGGL(stats_bf16_kernel<64>, grid, block, 0, stream, kk, vv, g.T, g.N,
                               second_order, out->kbar, out->vsum, out->ksig2, kc, vc, hpart);
    } else {
        auto kc = static_cast<float*>(out->kbar_c);
        auto vc = static_cast<float*>(out->vbar_c);
        auto kk = static_cast<const float*>(k);
        auto vv = static_cast<const float*>(v);
        if (g.D == 128)
            hipLaunchKernelGGL(stats_f32_kernel<128>, grid, block, 0, stream, kk, vv, g.T, g.N,
                               second_order, out->kbar, out->vsum, out->ksig2, kc, vc, hpart);
        else
            hipLaunchKernelGGL(stats_f32_kernel<64>, grid, block, 0, stream, kk, vv, g.T, g.N,
                               second_order, out->kbar, out->vsum, out->ksig2, kc, vc, hpart);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int DD = g.D * g.D;
    dim3 rgrid((DD + kThreads - 1) / kThreads, (unsigned)g.BH);
    hipLaunchKernelGGL(hsum_reduce_kernel, rgrid, block, 0, stream, hpart, G, DD, out->hsum);
    return hipGetLastError();
}

}  // namespace pisa
