// Fused PISA forward for fp32 inputs on the gfx950 fp32 matrix cores (PISA,
// §3.4 Algorithm 1 Phases 1-3, Eqs. 3-5 and 9-10; Piecewise-Taylor-Attention
// README for the gated second-order logit term).
//
// One workgroup (4 wave64) per (batch*head, 64-row query block i); wave w owns
// query rows 16 w .. 16 w + 15 of the block and all four waves walk the same
// items, so each item's K and V tiles are staged once in LDS and read by all
// of them. Items: the exact blocks of S_i in ascending order (band, sinks and
// routed ids, as a set), then the virtual-token groups (64 consecutive KV
// blocks each, a block of S_i or past N masked out).
//
// Per item and wave, v_mfma_f32_16x16x4_f32 (fp32 products, fp32 sums):
//   S^T = K Q'^T   A = K (16 keys x 4 dims) read from LDS, B = Q'^T held in
//                  registers for the whole block (q' = s log2(e) q, so the
//                  logits are in log2 units). Lane l holds query l % 16 and
//                  keys 16 kb + 4 (l / 16) + e of key tile kb. Lane group
//                  g = l / 16 carries head dims g D/4 .. g D/4 + D/4 - 1 in its
//                  k-slots (any bijection of the dims onto k-slots gives the
//                  same dot products), so each lane reads contiguous 16-byte
//                  chunks.
//   online softmax with rescaling (max over the row's 64 keys by two lane
//                  exchanges); P stays fp32.
//   O^T += V^T P   B = P straight from the S^T accumulator (k-step (kb, e)
//                  takes keys 16 kb + 4 g + e), A = V rows from LDS. Output
//                  tile dt row m is head dim 4 m + dt % 4 + 64 (dt / 4), so the
//                  A operand of a k-step is one or two 16-byte LDS reads.
// A virtual token j is a key k-bar_j with value V-hat_j (the block sum) and
// weight a = 2^(lam - m); its mass n_j a enters the row sum and the tail mass.
// Phase 3: G^T = H^T Q'^T on the same matrix cores (H rows from memory), and
// o = (acc + (l_tail / T) ln2 G) / l.
//
// LDS tiles hold rows of 16-byte chunks with chunk c of row r at position
// c ^ (r % 16): the K reads (16 rows, one chunk each) and the V reads (one
// row, 16 chunks) of 16 lanes then touch 16 distinct 16-byte bank groups.
#include <math.h>

#include "common.h"

namespace pisa {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;
constexpr int kMaxWordsF = 8192 / 32;          // selection bitmask words (N <= 8192)
constexpr uint32_t kRsrcWord3F = 0x00020000u;  // gfx9 raw buffer descriptor, dword 3

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_f32(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             (int)kRsrcWord3F);
}

// 16 bytes per lane from a buffer into LDS: lane l writes the LDS base + 16 l.
// Device pass only (the host pass rejects the builtin).
__device__ __forceinline__ void dma16_f32(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             (int)voff, 0, 0, 0);
#endif
}

__device__ __forceinline__ f32x4_t lds16(const unsigned char* p) {
    return *reinterpret_cast<const f32x4_t*>(p);
}

__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
struct CfgF {
    static constexpr int RB = 4 * D;          // row bytes
    static constexpr int CH = D / 4;          // 16-byte chunks per row
    static constexpr int TILE = 64 * RB;      // one 64-row tile
    static constexpr int RPI = 1024 / RB;     // rows per 1 KB DMA instruction
    static constexpr int NDMA = TILE / 1024;  // DMA instructions per tile
    static constexpr int QD = D / 4;          // dims (k-slots) per lane group
    static constexpr int DT = D / 16;         // 16-row output tiles
    static_assert(NDMA % 4 == 0, "DMA instructions split over the 4 waves");
};

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                     const double* __restrict__ kbar, const float* __restrict__ vsum,
                     const float* __restrict__ hsum, const int32_t* __restrict__ idx,
                     const float* __restrict__ wgate, float* __restrict__ o, float* __restrict__ rstat, int T,
                     int N, float scale, int topk, int band, int n_sink, int second_order, int first_order,
                     int phase_mask) {
    using C = CfgF<D>;
    // the two pipeline parities live in separate arrays so that the compiler
    // can tell the DMA into one from the reads of the other
    __shared__ __attribute__((aligned(16))) unsigned char kt0[C::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char kt1[C::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vt0[C::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char vt1[C::TILE];
    __shared__ uint32_t selbits[kMaxWordsF];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.y;
    const int i = blockIdx.x;
    const int r0 = i * kBlock;

    const bool do_exact = phase_mask == 0 || (phase_mask & 1);
    const bool do_virtual = phase_mask == 0 || (phase_mask & 2);
    const bool do_first = (phase_mask == 0 || (phase_mask & 4)) && first_order;

    // ---- selection bitmask of S_i (band, sinks, valid routed ids; a set)
    const int words = (N + 31) / 32;
    for (int w = tid; w < words; w += kThreads) selbits[w] = 0u;
    __syncthreads();
    {
        const Forced fs(i, band, n_sink, N);
        for (int c = tid; c < fs.count(); c += kThreads) {
            const int j = fs.block(c);
            atomicOr(&selbits[j >> 5], 1u << (j & 31));
        }
        const int32_t* row = topk > 0 ? idx + (bh * N + i) * (int64_t)topk : nullptr;
        for (int c = tid; c < topk; c += kThreads) {
            const int j = row[c];
            if (j >= 0 && j < N) atomicOr(&selbits[j >> 5], 1u << (j & 31));   // anything else is padding
        }
    }

    // ---- Q'^T operand: query row r0 + 16 wave + n16, dims g QD .. g QD + QD - 1
    const int tq = r0 + 16 * wave + n16;
    const float c2 = scale * kLog2eF;
    float qreg[C::QD];
    {
        const float* qr = q + (bh * T + (int64_t)min(tq, T - 1)) * D + g * C::QD;
#pragma unroll
        for (int c = 0; c < C::QD / 4; ++c) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t*>(qr + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) qreg[4 * c + e] = tq < T ? x[e] * c2 : 0.f;
        }
    }
    __syncthreads();

    const int GV = do_virtual ? (N + 63) / 64 : 0;
    const int nlast = T - (N - 1) * kBlock;     // rows of the last block
    // smallest selected block above j, or -1 (uniform LDS reads)
    auto next_set = [&](int j) -> int {
        int w = (j + 1) >> 5;
        if (w >= words) return -1;
        uint32_t b = selbits[w] & (~0u << ((j + 1) & 31));
        while (b == 0u) {
            if (++w >= words) return -1;
            b = selbits[w];
        }
        return 32 * w + __builtin_ctz(b);
    };
    // item codes: 0 .. N-1 an exact block, N + gi a virtual group, -1 the end
    auto next_item = [&](int it) -> int {
        if (it < N) {
            const int j = do_exact ? next_set(it) : -1;
            if (j >= 0) return j;
            return GV > 0 ? N : -1;
        }
        return it + 1 < N + GV ? it + 1 : -1;
    };

    // ---- staging of an item into the LDS tiles (all 256 threads)
    // DMA instruction n (wave n % 4) fills LDS bytes [1024 n, 1024 n + 1024):
    // lane l takes row RPI n + l / CH, position l % CH, which holds the row's
    // chunk (l % CH) ^ (row % 16).
    auto dma_tile = [&](const float* src, int rows, unsigned char* buf) {
        const __amdgpu_buffer_rsrc_t r = rsrc_f32(src, (uint32_t)(rows * C::RB));
#pragma unroll
        for (int n = wave; n < C::NDMA; n += 4) {
            const int rr = C::RPI * n + lane / C::CH, pos = lane % C::CH;
            dma16_f32(r, buf + 1024 * n, (uint32_t)(rr * C::RB + 16 * (pos ^ (rr & 15))));
        }
    };
    auto stage = [&](int it, unsigned char* kb, unsigned char* vb) {
        if (it < N) {
            const int64_t off = (bh * T + (int64_t)it * kBlock) * D;
            const int rows = min(kBlock, T - it * kBlock);
            dma_tile(k + off, rows, kb);
            dma_tile(v + off, rows, vb);
        } else {
            const int gi = it - N;
            const int rows = min(64, N - gi * 64);
            const int64_t off = (bh * N + (int64_t)gi * 64) * D;
            dma_tile(vsum + off, rows, vb);
            // k-bar rows (fp64) rounded to fp32; rows past N are zero
            for (int sl = tid; sl < 64 * C::CH; sl += kThreads) {
                const int rr = sl / C::CH, pos = sl % C::CH, ch = pos ^ (rr & 15);
                f32x4_t x = {0.f, 0.f, 0.f, 0.f};
                if (rr < rows) {
                    const double* s = kbar + off + (int64_t)rr * D + 4 * ch;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = (float)s[e];
                }
                *reinterpret_cast<f32x4_t*>(kb + rr * C::RB + 16 * pos) = x;
            }
        }
    };

    const float* wrow = second_order ? wgate + (bh * N + i) * (int64_t)N : nullptr;
    const float lnlast2 = log2f((float)nlast);

    float m = -INFINITY, lsum = 0.f, ltail = 0.f;   // per lane: partial sums over its keys
    f32x4_t acc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int it, const unsigned char* kb, const unsigned char* vb) {
        // S^T = K Q'^T: lane reads row 16 kt + n16 chunks g QD/4 + c
        f32x4_t s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C::QD / 4; ++c) {
            f32x4_t kv[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                const int rr = 16 * kt + n16;
                kv[kt] = lds16(kb + rr * C::RB + 16 * ((g * (C::QD / 4) + c) ^ (rr & 15)));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) s[kt] = mfma4(kv[kt][e], qreg[4 * c + e], s[kt]);
        }
        // logits (log2 units) with masks and biases; the max runs over the
        // mass exponents (virtual tokens: lam + log2 n_j)
        const bool virt = it >= N;
        float mx = -INFINITY;
        float wmass[4][4];   // virtual: n_j of each key (0 when masked)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = 16 * kt + 4 * g + e;
                float z = s[kt][e];
                if (!virt) {
                    if (key >= min(kBlock, T - it * kBlock)) z = -INFINITY;
                    mx = fmaxf(mx, z);
                    wmass[kt][e] = 1.f;
                } else {
                    const int j = (it - N) * 64 + key;
                    const bool ok = j < N && !((selbits[j >> 5] >> (j & 31)) & 1u);
                    if (ok && second_order) z += kLog2eF * wrow[j];
                    z = ok ? z : -INFINITY;
                    const float nj = j == N - 1 ? (float)nlast : 64.f;
                    mx = fmaxf(mx, z + (j == N - 1 ? lnlast2 : 6.f));
                    wmass[kt][e] = nj;
                }
                s[kt][e] = z;
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float cf = __builtin_amdgcn_exp2f(m - mu);   // 0 while nothing was seen
        m = mn;
        lsum *= cf;
        ltail *= cf;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[dt][e] *= cf;
        float add = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = __builtin_amdgcn_exp2f(s[kt][e] - mu);
                s[kt][e] = p;
                add = fmaf(p, wmass[kt][e], add);
            }
        lsum += add;
        if (virt) ltail += add;
        // O^T += V^T P: k-step (kt, e) takes keys 16 kt + 4 g' + e of lane group g'
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * kt + 4 * g + e;
                const unsigned char* vr = vb + rr * C::RB;
                const f32x4_t va = lds16(vr + 16 * (n16 ^ (rr & 15)));
#pragma unroll
                for (int d = 0; d < 4 && d < C::DT; ++d) acc[d] = mfma4(va[d], s[kt][e], acc[d]);
                if constexpr (C::DT > 4) {
                    const f32x4_t vb2 = lds16(vr + 16 * ((16 + n16) ^ (rr & 15)));
#pragma unroll
                    for (int d = 0; d < 4; ++d) acc[4 + d] = mfma4(vb2[d], s[kt][e], acc[4 + d]);
                }
            }
    };

    // ---- item pipeline: item n's tiles in parity n % 2, item n+1's DMA issued
    // after the barrier that ends every wave's reads of item n-1
    int cur = next_item(-1);
    if (cur >= 0) stage(cur, kt0, vt0);
    while (cur >= 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        int nxt = next_item(cur);
        if (nxt >= 0) stage(nxt, kt1, vt1);
        compute(cur, kt0, vt0);
        cur = nxt;
        if (cur < 0) break;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        nxt = next_item(cur);
        if (nxt >= 0) stage(nxt, kt0, vt0);
        compute(cur, kt1, vt1);
        cur = nxt;
    }

    // ---- row totals over the four lane groups
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    ltail += __shfl_xor(ltail, 16);
    ltail += __shfl_xor(ltail, 32);

    // ---- Phase 3: G^T = H^T Q'^T, same output layout as O^T
    if (do_first) {
        const float* H = hsum + bh * (int64_t)D * D;
        f32x4_t gacc[C::DT];
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) gacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int sidx = 0; sidx < C::QD; ++sidx) {
            const float* hr = H + (int64_t)(g * C::QD + sidx) * D + 4 * n16;
            const f32x4_t ha = *reinterpret_cast<const f32x4_t*>(hr);
#pragma unroll
            for (int d = 0; d < 4 && d < C::DT; ++d) gacc[d] = mfma4(ha[d], qreg[sidx], gacc[d]);
            if constexpr (C::DT > 4) {
                const f32x4_t hb = *reinterpret_cast<const f32x4_t*>(hr + 64);
#pragma unroll
                for (int d = 0; d < 4; ++d) gacc[4 + d] = mfma4(hb[d], qreg[sidx], gacc[4 + d]);
            }
        }
        const float fco = ltail > 0.f ? ltail / (float)T * kLn2F : 0.f;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[dt][e] = fmaf(fco, gacc[dt][e], acc[dt][e]);
    }

    // ---- o = acc / l: lane holds query tq, dims 16 g + 4 e + (0..3) (+ 64 for dt >= 4)
    if (tq < T) {
        const float inv = 1.f / lsum;
        float* orow = o + (bh * T + (int64_t)tq) * D;
#pragma unroll
        for (int h = 0; h < C::DT / 4; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f32x4_t x;
#pragma unroll
                for (int d = 0; d < 4; ++d) x[d] = acc[4 * h + d][e] * inv;
                *reinterpret_cast<f32x4_t*>(orow + 64 * h + 16 * g + 4 * e) = x;
            }
        if (rstat != nullptr && g == 0) {   // the row's lse and c
            const int64_t rr = 2 * (bh * (int64_t)T + tq);
            rstat[rr] = (m + log2f(lsum)) * kLn2F;
            rstat[rr + 1] = do_first ? ltail / lsum / (float)T : 0.f;
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const Geom& g, const pisa_params_t* p, const void* q, const void* k,
                               const void* v, const StatsView* st, const int32_t* idx, const float* wgate,
                               void* o, float* rstat, hipStream_t stream) {
    dim3 grid(g.N, (unsigned)g.BH), block(kThreads);
#define PISA_F32_LAUNCH(DD)                                                                          \
    hipLaunchKernelGGL((attn_f32_kernel<DD>), grid, block, 0, stream, static_cast<const float*>(q),  \
                       static_cast<const float*>(k), static_cast<const float*>(v), st->kbar, st->vsum, \
                       st->hsum, idx, wgate, static_cast<float*>(o), rstat, g.T, g.N, g.scale, p->topk, \
                       p->band, p->n_sink, p->second_order, p->first_order, p->phase_mask)
    if (g.D == 128) PISA_F32_LAUNCH(128);
    else PISA_F32_LAUNCH(64);
#undef PISA_F32_LAUNCH
    return hipGetLastError();
}

}  // namespace pisa
