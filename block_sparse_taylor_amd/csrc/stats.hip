// Prepare phase: block statistics of Q, K and V (PISA, Algorithm 1 step 1
// and Fig. 4 "Prepare Phase": block means Q-bar, K-bar, block value sums
// V-hat and the global first-order matrix H; Appendix C notation;
// Piecewise-Taylor-Attention README, "Blog post" for the per-dimension key
// variance and the pooled q^2, changelog "hc-free" statistics for
// sum_j (K_j - kbar_j)^T V_j = K^T V - sum_j kbar_j (x) V-hat_j).
//
// One workgroup streams BPW consecutive 64-row blocks of one (batch, head);
// the Q, K, V tiles of the next block are fetched while the current one is
// reduced, so Q, K and V are each read from HBM exactly once.
//   * Column statistics in fp64 (all 256 threads; each column's rows split
//     over the threads of that column, partials combined in LDS). Sums of
//     bf16 or fp32 inputs are exact in fp64, so the means equal a float64
//     evaluation bit for bit; the key variance uses sums shifted by the
//     block's first row (no cancellation against the mean).
//   * The partial first-order matrix sum_j (K_j^T V_j - kbar_j (x) V-hat_j):
//     bf16 inputs use bf16 MFMA (exact products, fp32 accumulation), fp32
//     inputs an fp64 VALU loop. Partials go to the workspace and a second
//     kernel adds those of a head in a fixed order (deterministic).
#include <algorithm>
#include <mutex>

#include "common.h"

namespace pisa {
namespace {

// Scratch of pisa_block_stats_noalloc (the partial H sums): a file-scope
// device array, one copy per GPU, held until the process ends. Host code
// never passes its name to a kernel (in host code the name is a host-side
// stand-in, not a device address); it uses the per-device address from
// hipGetSymbolAddress below.
__device__ __attribute__((aligned(256))) unsigned char scratch[PISA_STATS_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;

// Q, K, V are read once and the packed K copy is not read again by this
// kernel: both go through non-temporal loads / stores (measured: 322 -> 297 us
// at the Wan2.1-14B shape; either one alone gains little).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load(const void* p) {
    const nt_u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void nt_store(void* p, uint4 v) {
    __builtin_nontemporal_store((nt_u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u32x4*>(p));
}


// LDS row padding of the bf16 tiles (elements): a row pitch of 328 bytes
// (D = 128) or 200 (D = 64), an odd multiple of 8 bytes, so the 32 rows one
// packed-K read covers (8 bytes each) fall on distinct bank pairs, and the 4
// rows of a half-wave's transposed operand read overlap in few banks.
constexpr int kPad = 36;
// Blocks per workgroup: the (head, block range) workgroups of one call should
// all be resident at once. Two of these workgroups fit on a CU and MI355X has
// 256 CUs, so a head gets max(1, 512 / heads) ranges of at least 4 blocks
// (small problems still spread over the CUs; each range adds a D x D partial
// to write and reduce).
constexpr int kResidentWGs = 512;
constexpr int kMinBPW = 4;

struct StatsOut {
    double* qbar;
    double* q2bar;
    double* kbar;
    float* vsum;
    double* ksig2;
    void* kbar_c;
    void* vbar_c;
    void* kpack;      // bf16 only: K in the fused kernel's operand order
    void* kbpack;     // bf16 only: kbar_c in the same order, per group of 64 blocks
    bf16_t* kbar_r;   // kbar split bf16 hi + lo, in the router's MFMA operand order
    bf16_t* ksig2_r;  // second order: ksig2 the same way
    float* knorm;     // ||kbar_j||_2, rounded up
};

// ||kbar_j|| of block j from the fp32 means kb_s (wave 0; a visible kb_s),
// rounded up so that it bounds the fp64 norm: the router's error bound.
template <int D>
__device__ __forceinline__ void write_knorm(const float* kb_s, float* knorm, int64_t bh, int j, int N) {
    if (threadIdx.x >= 64) return;
    double s = 0.0;
    for (int d = threadIdx.x; d < D; d += 64) s = fma((double)kb_s[d], (double)kb_s[d], s);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (threadIdx.x == 0) knorm[bh * ((N + 15) / 16) * 16 + j] = (float)(sqrt(s) * (1.0 + 1e-6));
}

// Column statistics of one block from its LDS tiles (row pitch ld). The
// sums of squares (the pooled q'^2 and the key variances) only with the
// second-order term (SO).
template <typename T, int D, bool SO>
__device__ __forceinline__ void column_stats(const T* tq, const T* tk, const T* tv, int ld, int rows,
                                             int64_t bh, int j, int n_blocks, double s64,
                                             const StatsOut& out, double* red, float* kb_s,
                                             float* vs_s) {
    constexpr int H = kThreads / D;           // threads per column
    constexpr int RH = kBlock / H;            // rows per thread
    const int tid = threadIdx.x;
    const int c = tid % D, h = tid / D;
    const double shift = SO ? (double)load_f32(tk + c) : 0.0;   // block row 0 of this key column
    double sq = 0.0, sq2 = 0.0, sk = 0.0, skx = 0.0, skx2 = 0.0, sv = 0.0;
    const int n0 = h * RH, n1 = min(rows, n0 + RH);
    for (int n = n0; n < n1; ++n) {
        const double xq = (double)load_f32(tq + n * ld + c);
        const double xk = (double)load_f32(tk + n * ld + c);
        const double xv = (double)load_f32(tv + n * ld + c);
        sq += xq;
        sk += xk;
        sv += xv;
        if (SO) {
            const double yq = s64 * xq;
            sq2 += yq * yq;
            const double dk = xk - shift;
            skx += dk;
            skx2 += dk * dk;
        }
    }
    double* r = red + tid;
    r[0 * kThreads] = sq;
    r[2 * kThreads] = sk;
    r[5 * kThreads] = sv;
    if (SO) {
        r[1 * kThreads] = sq2;
        r[3 * kThreads] = skx;
        r[4 * kThreads] = skx2;
    }
    __syncthreads();
    if (tid < D) {
        double a[6];
#pragma unroll
        for (int s = 0; s < 6; ++s) {
            double x = 0.0;
            if (SO || s == 0 || s == 2 || s == 5) {
#pragma unroll
                for (int hh = 0; hh < H; ++hh) x += red[s * kThreads + hh * D + tid];
            }
            a[s] = x;
        }
        // x / rows; for a full block the exact product with 2^-6 (the same
        // correctly rounded value, without a division)
        const double n = (double)rows;
        auto per_row = [&](double x) { return rows == kBlock ? x * 0x1p-6 : x / n; };
        const double mean = per_row(a[2]);
        const int64_t off = (bh * n_blocks + j) * D;
        out.qbar[off + c] = per_row(a[0]);
        out.kbar[off + c] = mean;
        const int64_t rhead = bh * router_head_elems(n_blocks, D);
        router_store(out.kbar_r + rhead, j, c, D, mean);
        static_cast<T*>(out.kbar_c)[off + c] = store_cast<T>((float)mean);
        if (out.kbpack) {
            // block j = row j % 64 of virtual group j / 64, laid out like kpack
            const int r = j % 64;
            const int64_t gbase = (bh * ((n_blocks + 63) / 64) + j / 64) * (int64_t)(64 * D);
            static_cast<bf16_t*>(out.kbpack)[gbase + (((r / 32) * (D / 8) + c / 8) * 32 + r % 32) * 8 + c % 8] =
                f32_to_bf16((float)mean);
        }
        const float vs = (float)a[5];
        out.vsum[off + c] = vs;
        // the virtual token's value from the stored fp32 V-hat (as
        // prepare_operands_kernel forms it from a caller's statistics)
        static_cast<T*>(out.vbar_c)[off + c] = store_cast<T>((float)per_row((double)vs));
        kb_s[c] = (float)mean;
        vs_s[c] = (float)a[5];
        if (SO) {
            out.q2bar[off + c] = per_row(a[1]);
            const double mx = per_row(a[3]);
            const double s2 = fmax(per_row(a[4]) - mx * mx, 0.0);
            out.ksig2[off + c] = s2;
            router_store(out.ksig2_r + rhead, j, c, D, s2);
        }
    }
}

// ---------------------------------------------------------------- bf16 path (MFMA)
// An MFMA operand of 8 bf16 k-values from a row-major LDS tile (row pitch LD
// elements) by two transposed reads: lane l (tile column c0 + l % 32) gets
// rows r0 + 4 g + (0..3) and r0 + 8 + 4 g + (0..3), g = l / 32. Lanes address
// 4 consecutive elements of one row each: within a group of 16 lanes, lane
// 4 a + b reads row 4 g + a at columns 16 (l / 16 % 2) + 4 b .. + 3.
template <int LD>
__device__ __forceinline__ bf16x8_t tr_operand(const bf16_t* tile, int r0, int c0, int lane) {
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
    const int tri = lane & 15;
    const int row = r0 + 4 * (lane >> 5) + (tri >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (tri & 3);
    const bf16_t* p = tile + row * LD + col;
    const v4i16_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16_t y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 8 * LD));
    const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
    return __builtin_bit_cast(bf16x8_t, make_uint4(ux.x, ux.y, uy.x, uy.y));
}

// 32x32x16 bf16 MFMA operand layout (lane l, element e in 0..7):
//   A[m = l%32][k = 8(l/32) + e],  B[k = 8(l/32) + e][n = l%32]
//   C[m = 8(i/4) + 4(l/32) + i%4][n = l%32] for accumulator register i.
// C[a][b] += sum_t K[t][a] V[t][b]: A = K^T and B = V, both by transposed
// reads of the row-major LDS tiles (tr_operand; the k order of a k-step is
// permuted alike in both operands, which leaves the sum unchanged).
template <int D, bool SO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void stats_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v, int T,
    int N, int bpw, double s64, StatsOut out, float* __restrict__ hpart) {
    constexpr int LD = D + kPad;
    constexpr int CH = D / 8;                       // 16-byte chunks per row
    constexpr int LOADS = kBlock * CH / kThreads;   // uint4 loads per thread per tensor
    constexpr int NT = D / 32;                      // 32-wide tiles per dim
    constexpr int TPW = NT * NT / 4;                // output tiles per wave
    __shared__ __attribute__((aligned(16))) bf16_t sq[kBlock * LD];
    __shared__ __attribute__((aligned(16))) bf16_t sk[kBlock * LD];
    __shared__ __attribute__((aligned(16))) bf16_t sv[kBlock * LD];
    __shared__ double red[6 * kThreads];
    __shared__ float kb_s[D];
    __shared__ float vs_s[D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int j0 = g * bpw;
    const int j1 = min(N, j0 + bpw);
    const int64_t base = bh * (int64_t)T * D;

    f32x16_t acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

    uint4 pq[LOADS], pk[LOADS], pv[LOADS];
    auto fetch = [&](int j) {
#pragma unroll
        for (int L = 0; L < LOADS; ++L) {
            const int c = L * kThreads + tid;
            const int row = c / CH, ch = c % CH;
            const int t = j * kBlock + row;
            if (t < T) {
                const int64_t o = base + (int64_t)t * D + ch * 8;
                pq[L] = nt_load(q + o);
                pk[L] = nt_load(k + o);
                pv[L] = nt_load(v + o);
            } else {
                pq[L] = make_uint4(0, 0, 0, 0);
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
            const int o = row * LD + ch * 8;
            uint2* dq = reinterpret_cast<uint2*>(sq + o);
            uint2* dk = reinterpret_cast<uint2*>(sk + o);
            uint2* dv = reinterpret_cast<uint2*>(sv + o);
            dq[0] = make_uint2(pq[L].x, pq[L].y);
            dq[1] = make_uint2(pq[L].z, pq[L].w);
            dk[0] = make_uint2(pk[L].x, pk[L].y);
            dk[1] = make_uint2(pk[L].z, pk[L].w);
            dv[0] = make_uint2(pv[L].x, pv[L].y);
            dv[1] = make_uint2(pv[L].z, pv[L].w);
        }
        __syncthreads();
        if (j + 1 < j1) fetch(j + 1);

        // K of this block in the fused kernel's operand order: for each 32-row
        // half, the 16-byte chunks (8 dims) chunk-major, then row, so that one
        // 1 KB run holds a chunk pair of all 32 rows (rows past T are zero).
        {
            uint4* kp = reinterpret_cast<uint4*>(out.kpack) + (bh * N + j) * (int64_t)(kBlock * CH);
#pragma unroll
            for (int L = 0; L < LOADS; ++L) {
                const int c = L * kThreads + tid;
                const int half = c / (32 * CH), ch = (c / 32) % CH, r = c % 32;
                const uint2* src = reinterpret_cast<const uint2*>(sk + (32 * half + r) * LD + ch * 8);
                const uint2 lo = src[0], hi = src[1];
                nt_store(kp + c, make_uint4(lo.x, lo.y, hi.x, hi.y));
            }
        }

        // acc += K_j^T V_j  (rows >= `rows` are zero in LDS). Both operands by
        // the gfx950 transposed LDS read (ds_read_b64_tr_b16): lane l receives
        // column l % 32 of a 32-column tile at 4 consecutive rows; the two
        // reads of a 16-row k-step cover rows 4 (l / 32) + (0..3) and
        // 8 + 4 (l / 32) + (0..3), the same order of k for A = K^T and B = V.
        const int m = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < kBlock / 16; ++ks) {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int tile = wave * TPW + t;
                const int mt = tile / NT, nt = tile % NT;
                const bf16x8_t a = tr_operand<LD>(sk, ks * 16, mt * 32, lane);
                const bf16x8_t b = tr_operand<LD>(sv, ks * 16, nt * 32, lane);
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
            }
        }

        column_stats<bf16_t, D, SO>(sq, sk, sv, LD, rows, bh, j, N, s64, out, red, kb_s, vs_s);
        __syncthreads();  // kb_s / vs_s visible
        write_knorm<D>(kb_s, out.knorm, bh, j, N);
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

    // rows past the last block in the last virtual-key group are zero
    if (out.kbpack && j1 == N && N % 64 != 0) {
        const int GV = (N + 63) / 64;
        bf16_t* gp = static_cast<bf16_t*>(out.kbpack) + (bh * GV + GV - 1) * (int64_t)(64 * D);
        for (int e = tid; e < 64 * D; e += kThreads) {
            const int r = (e / (32 * D)) * 32 + (e / 8) % 32;   // row of packed element e
            if (r >= N % 64) gp[e] = 0;
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
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v, int T,
    int N, int bpw, int second_order, double s64, StatsOut out, float* __restrict__ hpart) {
    constexpr int LD = D + 1;
    constexpr int PER = D * D / kThreads;
    __shared__ float sq[kBlock * LD];
    __shared__ float sk[kBlock * LD];
    __shared__ float sv[kBlock * LD];
    __shared__ double red[6 * kThreads];
    __shared__ float kb_s[D];
    __shared__ float vs_s[D];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int g = blockIdx.x;
    const int j0 = g * bpw, j1 = min(N, j0 + bpw);
    const int64_t base = bh * (int64_t)T * D;
    double acc[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) acc[r] = 0.0;
    for (int j = j0; j < j1; ++j) {
        const int rows = min(kBlock, T - j * kBlock);
        __syncthreads();
        for (int c = tid; c < kBlock * D; c += kThreads) {
            const int row = c / D, col = c % D;
            const bool ok = row < rows;
            const int64_t o = base + ((int64_t)j * kBlock + row) * D + col;
            sq[row * LD + col] = ok ? q[o] : 0.f;
            sk[row * LD + col] = ok ? k[o] : 0.f;
            sv[row * LD + col] = ok ? v[o] : 0.f;
        }
        __syncthreads();
        if (second_order) column_stats<float, D, true>(sq, sk, sv, LD, rows, bh, j, N, s64, out, red, kb_s, vs_s);
        else column_stats<float, D, false>(sq, sk, sv, LD, rows, bh, j, N, s64, out, red, kb_s, vs_s);
        __syncthreads();  // kb_s visible
        write_knorm<D>(kb_s, out.knorm, bh, j, N);
        // partial H in fp64 from the exact products and exact column sums
#pragma unroll
        for (int r = 0; r < PER; ++r) {
            const int e = tid + r * kThreads;
            const int a = e / D, b = e % D;
            double s = 0.0, ka = 0.0, vb = 0.0;
            for (int n = 0; n < rows; ++n) {
                const double x = (double)sk[n * LD + a], y = (double)sv[n * LD + b];
                s += x * y;
                ka += x;
                vb += y;
            }
            acc[r] += s - ka * vb / (double)rows;
        }
    }
    float* hp = hpart + ((bh * gridDim.x) + g) * (int64_t)D * D;
#pragma unroll
    for (int r = 0; r < PER; ++r) hp[tid + r * kThreads] = (float)acc[r];
}

// H split into bf16 hi + lo in the fused kernel's MFMA A-operand order for
// G = Q H: element (dt, ks, part, lane, e) is the part of
// H[16 ks + 8 (lane / 32) + e][32 dt + lane % 32].
__device__ __forceinline__ void write_hpack(bf16_t* hpack, int64_t bh, int D, int e, float h) {
    const int DD = D * D;
    const int a = e / D, b = e % D;            // key dim, value dim
    const int dt = b / 32, lane = 32 * ((a % 16) / 8) + b % 32, ks = a / 16, el = a % 8;
    const int64_t o = bh * (int64_t)(2 * DD) + ((int64_t)((dt * (D / 16) + ks) * 2) * 64 + lane) * 8 + el;
    const bf16_t hi = f32_to_bf16(h);
    hpack[o] = hi;
    hpack[o + 64 * 8] = f32_to_bf16(h - bf16_to_f32(hi));
}

// Fixed-order sum of the per-workgroup partials of each head.
// Sums the partial H of a head in fixed order. For bf16 inputs it also writes
// H split into bf16 hi + lo in the fused kernel's MFMA A-operand order for
// G = Q H: element (dt, ks, part, lane, e) is the part of
// H[16 ks + 8 (lane / 32) + e][32 dt + lane % 32].
__global__ __launch_bounds__(kThreads) void hsum_reduce_kernel(const float* __restrict__ hpart,
                                                               int G, int D, float* __restrict__ hsum,
                                                               bf16_t* __restrict__ hpack) {
    const int64_t bh = blockIdx.y;
    const int DD = D * D;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= DD) return;
    const float* p = hpart + bh * (int64_t)G * DD + e;
    double s = 0.0;
    for (int g = 0; g < G; ++g) s += (double)p[(int64_t)g * DD];
    const float h = (float)s;
    hsum[bh * DD + e] = h;
    if (hpack) write_hpack(hpack, bh, D, e, h);
}

// The operand layouts from a caller's statistics (and K). Workgroup (j, bh)
// with j < N writes block j's entries, exactly as the statistics pass does
// from its own results; workgroup (N, bh) writes the head's hpack and the zero
// rows of the last virtual-key group.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void prepare_operands_kernel(
    const T* __restrict__ k, const double* __restrict__ kbar, const float* __restrict__ vsum,
    const double* __restrict__ ksig2, const float* __restrict__ hsum, int T_, int N, StatsOut out,
    bf16_t* __restrict__ hpack) {
    constexpr int CH = D / 8;
    constexpr int LD = D + 8;
    __shared__ __attribute__((aligned(16))) bf16_t sk[kBlock * LD];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int j = blockIdx.x;
    if (j == N) {
        if (hpack) {
            for (int e = tid; e < D * D; e += kThreads) write_hpack(hpack, bh, D, e, hsum[bh * D * D + e]);
        }
        if (out.kbpack && N % 64 != 0) {
            const int GV = (N + 63) / 64;
            bf16_t* gp = static_cast<bf16_t*>(out.kbpack) + (bh * GV + GV - 1) * (int64_t)(64 * D);
            for (int e = tid; e < 64 * D; e += kThreads) {
                const int r = (e / (32 * D)) * 32 + (e / 8) % 32;
                if (r >= N % 64) gp[e] = 0;
            }
        }
        return;
    }
    __shared__ float kb_s[D];
    const int rows = min(kBlock, T_ - j * kBlock);
    const int64_t off = (bh * N + j) * D;
    if (tid < D) {
        const int c = tid;
        const double mean = kbar[off + c];
        const int64_t rhead = bh * router_head_elems(N, D);
        router_store(out.kbar_r + rhead, j, c, D, mean);
        kb_s[c] = (float)mean;
        static_cast<T*>(out.kbar_c)[off + c] = store_cast<T>((float)mean);
        if (out.kbpack) {
            const int r = j % 64;
            const int64_t gbase = (bh * ((N + 63) / 64) + j / 64) * (int64_t)(64 * D);
            static_cast<bf16_t*>(out.kbpack)[gbase + (((r / 32) * (D / 8) + c / 8) * 32 + r % 32) * 8 + c % 8] =
                f32_to_bf16((float)mean);
        }
        static_cast<T*>(out.vbar_c)[off + c] = store_cast<T>((float)((double)vsum[off + c] / (double)rows));
        if (out.ksig2_r) router_store(out.ksig2_r + rhead, j, c, D, ksig2[off + c]);
    }
    __syncthreads();
    write_knorm<D>(kb_s, out.knorm, bh, j, N);
    if (out.kpack) {
        // the block's K rows through LDS (coalesced loads), then in packed order
        const bf16_t* kh = reinterpret_cast<const bf16_t*>(k) + bh * (int64_t)T_ * D;
        for (int c = tid; c < kBlock * CH; c += kThreads) {
            const int row = c / CH, ch = c % CH;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (row < rows) u = *reinterpret_cast<const uint4*>(kh + ((int64_t)j * kBlock + row) * D + 8 * ch);
            *reinterpret_cast<uint4*>(sk + row * LD + 8 * ch) = u;
        }
        __syncthreads();
        uint4* kp = reinterpret_cast<uint4*>(out.kpack) + (bh * N + j) * (int64_t)(kBlock * CH);
        for (int c = tid; c < kBlock * CH; c += kThreads) {
            const int half = c / (32 * CH), ch = (c / 32) % CH, r = c % 32;
            kp[c] = *reinterpret_cast<const uint4*>(sk + (32 * half + r) * LD + 8 * ch);
        }
    }
}

int stats_bpw(const Geom& g) {
    int64_t groups = std::max<int64_t>(1, kResidentWGs / g.BH);
    groups = std::min<int64_t>(groups, (g.N + kMinBPW - 1) / kMinBPW);
    return (int)((g.N + groups - 1) / groups);
}

int stats_groups(const Geom& g) {
    const int bpw = stats_bpw(g);
    return (g.N + bpw - 1) / bpw;
}

}  // namespace

hipError_t stats_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with this device current
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

size_t stats_workspace_bytes_for(const Geom& g, int cov_bias) {
    const size_t part = (size_t)g.BH * stats_groups(g) * g.D * g.D * sizeof(float);
    return cov_bias ? std::max(part, cov_workspace_bytes(g, stats_groups(g))) : part;
}

size_t stats_workspace_bytes(const Geom& g) { return stats_workspace_bytes_for(g, 1); }

hipError_t launch_prepare_operands(const Geom& g, int dtype, int second_order, const void* k,
                                   const StatsView* st, hipStream_t stream) {
    const bool bf = dtype == PISA_BF16;
    StatsOut out{nullptr, nullptr, nullptr, nullptr, nullptr, st->kbar_c, st->vbar_c,
                 bf ? st->kpack : nullptr, bf ? st->kbpack : nullptr, st->kbar_r,
                 second_order ? st->ksig2_r : nullptr, st->knorm};
    bf16_t* hp = bf ? static_cast<bf16_t*>(st->hpack) : nullptr;
    const dim3 grid(g.N + 1, (unsigned)g.BH), block(kThreads);
#define PISA_PREP_LAUNCH(TT, DD)                                                                   \
    hipLaunchKernelGGL((prepare_operands_kernel<TT, DD>), grid, block, 0, stream,                 \
                       static_cast<const TT*>(k), st->kbar, st->vsum, second_order ? st->ksig2 : nullptr, \
                       st->hsum, g.T, g.N, out, hp)
    if (bf) {
        if (g.D == 128) PISA_PREP_LAUNCH(bf16_t, 128);
        else PISA_PREP_LAUNCH(bf16_t, 64);
    } else {
        if (g.D == 128) PISA_PREP_LAUNCH(float, 128);
        else PISA_PREP_LAUNCH(float, 64);
    }
#undef PISA_PREP_LAUNCH
    return hipGetLastError();
}

hipError_t launch_block_stats(const Geom& g, int dtype, int second_order, int cov_bias, const void* q,
                              const void* k, const void* v, const StatsView* st, void* workspace,
                              hipStream_t stream) {
    const int G = stats_groups(g), bpw = stats_bpw(g);
    dim3 grid(G, (unsigned)g.BH), block(kThreads);
    float* hpart = static_cast<float*>(workspace);
    StatsOut out{st->qbar, st->q2bar, st->kbar, st->vsum, st->ksig2, st->kbar_c, st->vbar_c, st->kpack,
                 dtype == PISA_BF16 ? st->kbpack : nullptr, st->kbar_r,
                 second_order ? st->ksig2_r : nullptr, st->knorm};
#define PISA_STATS_BF16(DD, SO)                                                                    \
    hipLaunchKernelGGL((stats_bf16_kernel<DD, SO>), grid, block, 0, stream,                       \
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),              \
                       static_cast<const bf16_t*>(v), g.T, g.N, bpw, g.scale64, out, hpart)
#define PISA_STATS_F32(DD)                                                                         \
    hipLaunchKernelGGL(stats_f32_kernel<DD>, grid, block, 0, stream, static_cast<const float*>(q), \
                       static_cast<const float*>(k), static_cast<const float*>(v), g.T, g.N, bpw, \
                       second_order, g.scale64, out, hpart)
    if (dtype == PISA_BF16) {
        if (g.D == 128) {
            if (second_order) PISA_STATS_BF16(128, true);
            else PISA_STATS_BF16(128, false);
        } else {
            if (second_order) PISA_STATS_BF16(64, true);
            else PISA_STATS_BF16(64, false);
        }
    } else {
        if (g.D == 128) PISA_STATS_F32(128);
        else PISA_STATS_F32(64);
    }
#undef PISA_STATS_BF16
#undef PISA_STATS_F32
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int DD = g.D * g.D;
    dim3 rgrid((DD + kThreads - 1) / kThreads, (unsigned)g.BH);
    hipLaunchKernelGGL(hsum_reduce_kernel, rgrid, block, 0, stream, hpart, G, g.D, st->hsum,
                       dtype == PISA_BF16 ? static_cast<bf16_t*>(st->hpack) : nullptr);
    e = hipGetLastError();
    if (e != hipSuccess || !cov_bias) return e;
    // the covariance prior's block norms, after the block means (same workspace)
    return launch_cov_norm(g, dtype, k, v, st->kbar, st->hnorm, workspace, G, stream);
}

}  // namespace pisa
