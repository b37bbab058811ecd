// Routing: top-k KV blocks per query block from pooled block scores (PISA,
// Algorithm 1 step 2, the block score of Eq. 11 without its covariance term;
// Piecewise-Taylor-Attention README: +-band forced exact, clamped ranking
// spread min(w, ln B), set-identical top-k).
//
//   r_ij = s qbar_i . kbar_j  [+ min(w_ij, ln B)]  [+ log(M_j + eps)],
//   w_ij = 1/2 q2bar_i . ksig2_j,  M_j = hnorm_j (the covariance-aware prior of
//   PISA Eq. 11, when asked for)
//   Top_i = the topk largest r_ij over |i - j| > band and j >= n_sink (the
//   band and the README's sink blocks are forced exact), ties to the lower j.
//
// The decision must equal a float64 evaluation, so the kernel scores in fp32
// and settles every close call in fp64:
//   1. One workgroup per (batch*head, 16 query blocks). bf16 MFMA
//      (16x16x32) on the fp64 pooled statistics split into bf16 hi + lo
//      (three products per k-step) computes the 16 x N fp32 score rows into
//      LDS. |r~ - r| <= eps_i with a rigorous bound eps_i = (4 (3 D + 8) u +
//      4 2^-18) (s ||qbar_i|| max_j ||kbar_j|| [+ ln B] [+ max |prior|]).
//   2. Per row (one wave), a search over order-preserving 32-bit keys
//      (wave_select32) brackets tau~, the topk-th largest r~, within eps.
//      Blocks with r~ above the bracket by 2 eps are in Top_i, below it by
//      2 eps out; the few in between (close calls) are ranked exactly: each
//      one's r_ij is recomputed once in fp64 and the remaining members are
//      those of smallest rank (ties: lower j). Rows with more than kAmbCap
//      close calls use a 64-bit radix select over the fp64 scores instead.
//   3. Ids are written ascending, -1 padded.
// The gate of the second-order term is decided the same way (fp32, with an
// fp64 recomputation within the error bound of ln B) and the gated w table is
// written for the fused kernel. No N x N score matrix leaves the chip.
#include <math.h>

#include "common.h"

namespace pisa {
namespace {

constexpr int kQB = 16;               // query blocks per workgroup
constexpr int kAmbCap = 64;           // close calls ranked pairwise per row (more: radix select)
constexpr int kLdsMax = 160 * 1024;   // LDS of a gfx950 workgroup
constexpr int kLdsStatic = 256;        // at most this much static LDS beside the dynamic part
constexpr double kU = 5.9604644775390625e-08;   // 2^-24

// The covariance prior of block j, in fp64 (the same expression everywhere a
// score is formed, so fp32 and fp64 scores see the same value).
__device__ __forceinline__ double cov_prior(const double* hn, int j) { return log(hn[j] + PISA_COV_EPS); }

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4_t;
typedef double d2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t key32(float f) {
    f = f + 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u >> 31) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unkey32(uint32_t k) {
    return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ uint64_t key64(double r) {
    r = r + 0.0;
    const uint64_t u = __double_as_longlong(r);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Wave-wide inclusive prefix sum (lanes ascending).
__device__ __forceinline__ int wave_scan(int x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Radix select over one wave: the need-th largest key among those for which
// `take(j)` holds, j in [0, n); keys from key(j). Returns the key and, through
// need_eq, how many keys equal to it belong to the selection. hist: 256
// unsigned per wave in LDS.
template <typename Key, int BITS, typename KeyFn, typename TakeFn>
__device__ __forceinline__ Key wave_radix_select(int n, int need, KeyFn key, TakeFn take,
                                                 unsigned* hist, int* need_eq) {
    const int lane = threadIdx.x & 63;
    Key prefix = 0;
    for (int pass = 0; pass < BITS / 8; ++pass) {
        const int shift = BITS - 8 - 8 * pass;
        const Key hmask = pass == 0 ? (Key)0 : (Key)(~(Key)0 << (shift + 8));
#pragma unroll
        for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0u;
        __builtin_amdgcn_wave_barrier();
        for (int j = lane; j < n; j += 64) {
            if (!take(j)) continue;
            const Key kk = key(j);
            if ((kk & hmask) == prefix) atomicAdd(&hist[(unsigned)((kk >> shift) & 255)], 1u);
        }
        __builtin_amdgcn_wave_barrier();
        // lane L owns bins 255-4L .. 252-4L (top bins first)
        int c[4], s = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            c[b] = (int)hist[255 - 4 * lane - b];
            s += c[b];
        }
        const int incl = wave_scan(s);
        const int excl = incl - s;
        const unsigned long long hit = __ballot(incl >= need);
        const int L = __ffsll((long long)hit) - 1;       // first lane reaching need
        int digit = 0, rest = need;
        if (lane == L) {
            rest = need - excl;
            int b = 0;
            for (; b < 3; ++b) {
                if (c[b] >= rest) break;
                rest -= c[b];
            }
            digit = 255 - 4 * lane - b;
        }
        digit = __shfl(digit, L);
        need = __shfl(rest, L);
        prefix |= (Key)digit << shift;
        __builtin_amdgcn_wave_barrier();
    }
    *need_eq = need;
    return prefix;
}

// The need-th largest of the wave's 32-bit keys (KPL per lane, in registers;
// 0 marks an excluded slot, below every real key), to within `width` in value.
// The search keeps a key interval [L, H] that holds the answer, with
// cL = #keys >= L >= need > cH = #keys > H, and probes one key c in (L, H]
// per step, counting the keys >= c with ballots (no atomics). The probe is
// a false-position step on the counts: the value at which a uniform spread
// of the keys between unkey(L) and unkey(H) would put the need-th largest,
// with the Illinois rule (an end kept twice in a row has its rank distance
// halved, so both ends move); after 24 steps the probes are value midpoints.
// A probe that would not split the interval is replaced by the key midpoint.
// It stops when the interval spans at most `width` in value (the caller
// settles everything within its error bound of the interval exactly), when
// L = H, or when exactly `need` keys reach L (the answer is then the smallest
// of them, a wave minimum). Real keys are those of finite floats, so unkey()
// of any key in [L, H] is finite. Returns the interval in *lo, *hi.
constexpr int kKeysPerLane = 36;       // the fast kernel's rows: N <= 64 * 36
template <int KPL>
__device__ __forceinline__ void wave_select32(const uint32_t (&kv)[KPL], int need, float width, uint32_t* lo,
                                              uint32_t* hi) {
    auto count_ge = [&](uint32_t c) {
        int n = 0;
#pragma unroll
        for (int i = 0; i < KPL; ++i) n += __popcll(__ballot(kv[i] >= c));
        return n;
    };
    auto min_ge = [&](uint32_t c) {   // the smallest key >= c, a wave minimum
        uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
        for (int i = 0; i < KPL; ++i) mn = kv[i] >= c ? min(mn, kv[i]) : mn;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
        return mn;
    };
    uint32_t mx = 0u;
#pragma unroll
    for (int i = 0; i < KPL; ++i) mx = max(mx, kv[i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    uint32_t L = min_ge(1u), H = mx;   // the smallest and largest real keys
    int cL = count_ge(L), cH = 0;
    float wl = 1.f, wh = 1.f;   // Illinois weights of the two ends' rank distances
    int last = 0;               // the end the previous step moved: 1 = L, 2 = H
    for (int step = 0; step < 80; ++step) {
        if (cL == need) {
            *lo = *hi = min_ge(L);
            return;
        }
        if (L == H) break;
        const float fl = unkey32(L), fh = unkey32(H);
        if (fh - fl <= width) break;
        float x;
        if (step < 24) {
            const float dl = (float)(cL - need) * wl, dh = (float)(need - cH) * wh;
            x = fh - (fh - fl) * (dh / (dl + dh));
        } else {
            x = 0.5f * fl + 0.5f * fh;
        }
        uint32_t c = key32(x);
        if (c <= L || c > H) c = L + ((H - L) >> 1) + 1u;   // progress: L < c <= H
        const int n = count_ge(c);
        if (n >= need) {
            L = c;
            cL = n;
            wh = last == 1 ? 0.5f * wh : 1.f;
            wl = 1.f;
            last = 1;
        } else {
            H = c - 1u;
            cH = n;
            wl = last == 2 ? 0.5f * wl : 1.f;
            wh = 1.f;
            last = 2;
        }
    }
    *lo = L;
    *hi = H;
}

// LDS of the fast kernel: the fp64 pooled q'^2 rows (second order only), fp32
// score rows of pitch NP, per-wave radix histograms, close-call lists and
// taken-bit masks. At N = 512 without the second order it is 39.3 KB, so four
// workgroups share a CU.
__host__ __device__ inline int fast_np(int N) { return (N + 3) & ~3; }
__host__ __device__ inline size_t fast_lds_bytes(int D, int N, int second_order, int nwv) {
    const int NP = fast_np(N);
    return (size_t)8 * kQB * D * (second_order ? 1 : 0) + (size_t)4 * kQB * NP + (size_t)nwv * 4 * 256 +
           (size_t)nwv * kAmbCap * (4 + 8) + (size_t)4 * nwv * ((NP + 31) / 32);
}
// Waves per workgroup: eight (two per SIMD), each taking two of the 16 score
// rows. Rows of more than 1024 blocks fill most of the LDS (one workgroup per
// CU); shorter rows fit two workgroups per CU, and smaller workgroups leave a
// shorter tail than four-wave ones (measured at N = 512: 118 -> 112 us with
// 40 heads, 63 -> 54 us with 12, FLUX 45 -> 34 us; same routing).
__host__ __device__ constexpr int route_waves(int) { return 8; }

// KPL: keys per lane of a score row (N <= 64 KPL); rows of up to 1024 blocks
// without the second order fit four waves per SIMD.
template <int D, bool SO, int KPL, bool COV>
__global__ __launch_bounds__(64 * route_waves(KPL)) __attribute__((amdgpu_waves_per_eu(SO || KPL > 16 ? 2 : 4))) void route_fast_kernel(
    const double* __restrict__ qbar, const double* __restrict__ q2bar, const double* __restrict__ kbar,
    const bf16_t* __restrict__ kbar_r, const double* __restrict__ ksig2, const bf16_t* __restrict__ ksig2_r,
    const float* __restrict__ knorm, const double* __restrict__ hnorm, int N, double s64, int topk, int band,
    int n_sink,
    int32_t* __restrict__ idx, float* __restrict__ wgate) {
    constexpr int KS = D / 4;       // 16x16x4 k-steps; MFMA k-slot (ks, l/16) <-> dim (D/4)(l/16) + ks
    constexpr bool second_order = SO;
    constexpr int NWV = route_waves(KPL), NT = 64 * NWV;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int NP = fast_np(N), NW = (NP + 31) / 32;
    double* q2_s = reinterpret_cast<double*>(lds);                   // second order only
    float* score_s = reinterpret_cast<float*>(q2_s + (second_order ? kQB * D : 0));
    unsigned* hist_s = reinterpret_cast<unsigned*>(score_s + kQB * NP);
    int* amb_j_s = reinterpret_cast<int*>(hist_s + NWV * 256);
    double* amb_r_s = reinterpret_cast<double*>(amb_j_s + NWV * kAmbCap);
    uint32_t* take_s = reinterpret_cast<uint32_t*>(amb_r_s + NWV * kAmbCap);
    __shared__ float kmax_s[NWV];
    __shared__ float bmax_s[NWV];
    static_assert(2 * 4 * NWV <= kLdsStatic, "static LDS beyond the launcher's reserve");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t bh = blockIdx.y;
    const int i0 = blockIdx.x * kQB;
    const int nq = min(kQB, N - i0);
    const double lnB = log((double)kBlock);
    const float lnBf = (float)lnB;

    // pooled q'^2 of the tile's query blocks (zeros past N), second order only
    if (second_order) {
        for (int e = tid; e < kQB * D; e += NT) {
            const int r = e / D;
            q2_s[e] = r < nq ? q2bar[(bh * N + i0 + r) * (int64_t)D + e % D] : 0.0;
        }
        __syncthreads();
    }
    const double* qrows = qbar + (bh * N + i0) * (int64_t)D;   // fp64 pooled queries of the tile
    // the pooled query of each row this wave selects for (dims 2 lane, 2 lane
    // + 1), loaded now so that the loads overlap the score products (with the
    // covariance prior, whose kernels hold fewer free registers, per row)
    constexpr int RPW = COV ? 1 : (kQB + NWV - 1) / NWV;   // rows per wave preloaded
    auto load_q = [&](int r) {
        d2_t x = {0.0, 0.0};
        if (r < nq && 2 * lane < D) x = *reinterpret_cast<const d2_t*>(qrows + (int64_t)r * D + 2 * lane);
        return x;
    };
    d2_t qpre[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) qpre[rr] = COV ? d2_t{0.0, 0.0} : load_q(wave + rr * NWV);

    // ---- scores: S[r][j] = s qbar_r . kbar_j (+ min(w, ln B)) (+ prior) via
    // bf16 MFMA 16x16x32 on operands split into hi + lo (hi.hi + hi.lo + lo.hi:
    // what is dropped is below 3.01 2^-18 of each |q_d k_d|, and the products are
    // exact in fp32). Wave w takes the 16-column chunks c = w, w+NWV, ...; lane
    // (m16, g4) holds k-slots 8 g4 + e of k-step s for dim (D/4) g4 + 8 s + e:
    // for the A operand the pooled query row m16, for B key 16 c + m16, which
    // kbar_r holds as 2 (D/32) 1 KB runs per chunk, loaded one chunk ahead.
    constexpr int KB = D / 32;      // bf16 16x16x32 k-steps
    const int m16 = lane & 15, g4 = lane >> 4;
    auto split8 = [&](const double* x, bool valid, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const double v = valid ? x[e] : 0.0;
            const __bf16 h = (__bf16)(float)v;
            hi[e] = h;
            lo[e] = (__bf16)(float)(v - (double)(float)h);
        }
    };
    bf16x8_t ah[KB], al[KB], a2h[SO ? KB : 1], a2l[SO ? KB : 1];
    {
        const double* qa = qrows + min(m16, nq - 1) * D + (D / 4) * g4;
#pragma unroll
        for (int sk = 0; sk < KB; ++sk) split8(qa + 8 * sk, m16 < nq, ah[sk], al[sk]);
        if (SO) {
#pragma unroll
            for (int sk = 0; sk < KB; ++sk) split8(q2_s + m16 * D + (D / 4) * g4 + 8 * sk, true, a2h[sk], a2l[sk]);
        }
    }
    const double* kb = kbar + bh * (int64_t)N * D;
    const double* sg = SO ? ksig2 + bh * (int64_t)N * D : nullptr;
    const double* hn = COV ? hnorm + bh * (int64_t)N : nullptr;   // covariance prior
    float kmaxf = 0.f;
    float bmax = 0.f;   // max |prior| over this wave's columns (of the fp32 roundings)
    const int NC = (N + 15) / 16;
    const uint4* kr4 = reinterpret_cast<const uint4*>(kbar_r + bh * router_head_elems(N, D));
    const uint4* sr4 = SO ? reinterpret_cast<const uint4*>(ksig2_r + bh * router_head_elems(N, D)) : nullptr;
    const float* kn = knorm + bh * (int64_t)NC * 16;
    uint4 kv[2 * KB], sv[SO ? 2 * KB : 1];   // this chunk's B operands (key means; variances)
    auto kload = [&](int c) {   // one chunk ahead of its MFMAs
#pragma unroll
        for (int u = 0; u < 2 * KB; ++u) kv[u] = kr4[((int64_t)c * 2 * KB + u) * 64 + lane];
        if (SO) {
#pragma unroll
            for (int u = 0; u < 2 * KB; ++u) sv[u] = sr4[((int64_t)c * 2 * KB + u) * 64 + lane];
        }
    };
    if (wave < NC) kload(wave);
    for (int c = wave; c < NC; c += NWV) {
        const int col = c * 16 + m16;
        const bool ok = col < N;
        bf16x8_t bh8[KB], bl8[KB], sh8[SO ? KB : 1], sl8[SO ? KB : 1];
#pragma unroll
        for (int sk = 0; sk < KB; ++sk) {
            bh8[sk] = __builtin_bit_cast(bf16x8_t, ok ? kv[2 * sk] : make_uint4(0, 0, 0, 0));
            bl8[sk] = __builtin_bit_cast(bf16x8_t, ok ? kv[2 * sk + 1] : make_uint4(0, 0, 0, 0));
            if (SO) {
                sh8[sk] = __builtin_bit_cast(bf16x8_t, ok ? sv[2 * sk] : make_uint4(0, 0, 0, 0));
                sl8[sk] = __builtin_bit_cast(bf16x8_t, ok ? sv[2 * sk + 1] : make_uint4(0, 0, 0, 0));
            }
        }
        if (c + NWV < NC) kload(c + NWV);   // the next chunk
        if (ok) kmaxf = fmaxf(kmaxf, kn[col]);
        f4_t acc = {0.f, 0.f, 0.f, 0.f}, accw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sk = 0; sk < KB; ++sk) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[sk], bh8[sk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[sk], bl8[sk], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[sk], bh8[sk], acc, 0, 0, 0);
        }
        if (SO) {
#pragma unroll
            for (int sk = 0; sk < KB; ++sk) {
                accw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2h[sk], sh8[sk], accw, 0, 0, 0);
                accw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2h[sk], sl8[sk], accw, 0, 0, 0);
                accw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2l[sk], sh8[sk], accw, 0, 0, 0);
            }
        }
        float prior = 0.f;
        if (COV && ok) {
            prior = (float)cov_prior(hn, col);
            bmax = fmaxf(bmax, fabsf(prior));
        }
        // C layout: lane holds column m16, rows 4 g4 + e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 4 * g4 + e;
            float sc = (float)s64 * acc[e];
            if (SO) {
                const bool live = ok && r < nq;
                const float w = 0.5f * accw[e];
                // all terms of w are >= 0: relative bound (split + fp32 sums)
                const float ew = (float)(2.0 * (3 * D + 4) * kU + 8.0 * 0x1p-18) * w + 1e-30f;
                const bool close = live && !(fabsf(w - lnBf) > ew);
                float wg = w > lnBf ? 0.f : w;
                // the few pairs too close to call in fp32 are decided in fp64, one
                // at a time by the whole wave (each lane two dims, a wave sum)
                unsigned long long cm = __ballot(close);
                while (cm) {
                    const int L = __ffsll((long long)cm) - 1;
                    cm &= cm - 1;
                    const int rr = 4 * (L >> 4) + e, cc = c * 16 + (L & 15);
                    double part = 0.0;
                    if (2 * lane < D) {
                        const d2_t y = *reinterpret_cast<const d2_t*>(sg + (int64_t)cc * D + 2 * lane);
                        part = fma(q2_s[rr * D + 2 * lane], y.x, q2_s[rr * D + 2 * lane + 1] * y.y);
                    }
#pragma unroll
                    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
                    const double w64 = 0.5 * part;
                    if (lane == L) wg = w64 > lnB ? 0.f : (float)w64;
                }
                if (live) {
                    wgate[(bh * N + i0 + r) * (int64_t)N + col] = wg;
                    sc += fminf(w, lnBf);
                }
            }
            sc += prior;
            if (ok) score_s[r * NP + col] = sc;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        kmaxf = fmaxf(kmaxf, __shfl_xor(kmaxf, off));
        bmax = fmaxf(bmax, __shfl_xor(bmax, off));
    }
    if (lane == 0) {
        kmax_s[wave] = kmaxf;
        bmax_s[wave] = bmax;
    }
    __syncthreads();
    float kmx = kmax_s[0];
    float bmxf = bmax_s[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
        kmx = fmaxf(kmx, kmax_s[w]);
        bmxf = fmaxf(bmxf, bmax_s[w]);
    }
    const double bmx = (double)bmxf * (1.0 + 1e-6);   // bounds |prior| in fp64 too
    const double kmax = (double)kmx;                  // the norms are rounded up already

    // ---- selection: wave w handles rows w, w+NWV, ... A row's candidate
    // keys stay in registers (lane l holds columns 64 i + l, i < KPL) from the
    // threshold search through the classification and the ascending write.
    unsigned* hist = hist_s + wave * 256;
    int* amb_j = amb_j_s + wave * kAmbCap;
    double* amb_r = amb_r_s + wave * kAmbCap;
    uint32_t* tbits = take_s + wave * NW;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    auto row_pass = [&](int r, d2_t qpair) {   // qpair: dims 2 lane, 2 lane + 1 of the row's pooled query
        const int i = i0 + r;
        int32_t* out = idx + (bh * N + i) * (int64_t)topk;
        const Forced fs(i, band, n_sink, N);
        const int ncand = N - fs.count();
        const int k = min(topk, ncand);
        const float* sr = score_s + r * NP;
        const double* qg = qrows + (int64_t)r * D;   // fp64 pooled query of row i
        auto is_cand = [&](int j) { return !fs.forced(j); };
        int written = 0;
        if (k > 0) {
            uint32_t kv[KPL];
#pragma unroll
            for (int t = 0; t < KPL; ++t) {
                const int j = 64 * t + lane;
                const float x = sr[min(j, N - 1)];
                kv[t] = j < N && is_cand(j) ? key32(x) : 0u;
            }
            double qn = fma(qpair.x, qpair.x, qpair.y * qpair.y);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) qn += __shfl_xor(qn, off);
            // |r| bound: the dot product, the clamped spread, the prior (the
            // latter two each add at most two fp32 roundings of their size)
            const double bound = s64 * sqrt(qn) * kmax + (second_order ? lnB : 0.0) + bmx;
            // fp32 sums of 3 D exact products (and of the spread and prior), plus
            // the split's dropped terms: |r~ - r| <= eps
            const float eps = (float)((4.0 * (3 * D + 8) * kU + 4.0 * 0x1p-18) * bound) + 1e-30f;
            uint32_t tlo, thi;
            wave_select32<KPL>(kv, k, eps, &tlo, &thi);
            // the k-th largest fp32 score lies in [unkey(tlo), unkey(thi)]; the band
            // around it in key space: x > hi <=> key > khi, x >= lo <=> key >= klo
            const uint32_t khi = key32(unkey32(thi) + 2.f * eps), klo = key32(unkey32(tlo) - 2.f * eps);
            // certain members (above the band) and the close calls inside it,
            // the latter listed in ascending j
            int cg = 0, ca = 0;
#pragma unroll
            for (int t = 0; t < KPL; ++t) {
                const bool in = kv[t] > khi;
                const bool amb = !in && kv[t] >= klo && kv[t] != 0u;
                cg += __popcll(__ballot(in));
                const unsigned long long am = __ballot(amb);
                const int pos = ca + __popcll(am & lt_mask);
                if (amb && pos < kAmbCap) amb_j[pos] = 64 * t + lane;
                ca += __popcll(am);
            }
            const int need = k - cg;      // members still to choose among the close calls
            auto exact = [&](int j) {     // fp64 score of block j
                const double* kr = kb + (int64_t)j * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot = fma(qg[d], kr[d], dot);
                double rr = s64 * dot;
                if (second_order) {
                    const double* sq = sg + (int64_t)j * D;
                    double w = 0.0;
                    for (int d = 0; d < D; ++d) w = fma(q2_s[r * D + d], sq[d], w);
                    rr += fmin(0.5 * w, lnB);
                }
                if (COV) rr += cov_prior(hn, j);
                return rr;
            };
            // the same score with the whole wave on one block: each lane takes
            // two dims (one 16-byte load, contiguous across lanes), then a
            // wave reduction (the fp64 sum in another order; decisions stay
            // those of float64 up to near-exact ties)
            // CB close calls at a time: all their loads first, then the
            // products and the wave sums (two with the covariance prior,
            // whose kernels hold fewer free registers)
            constexpr int CB = COV ? 2 : 4;
            auto exact_batch = [&](const int (&j)[CB], double (&rr)[CB]) {
                d2_t x[CB], y[CB];
#pragma unroll
                for (int u = 0; u < CB; ++u) {
                    x[u] = y[u] = d2_t{0.0, 0.0};
                    if (2 * lane < D) {
                        x[u] = *reinterpret_cast<const d2_t*>(kb + (int64_t)j[u] * D + 2 * lane);
                        if (second_order) y[u] = *reinterpret_cast<const d2_t*>(sg + (int64_t)j[u] * D + 2 * lane);
                    }
                }
                double dot[CB], w[CB];
#pragma unroll
                for (int u = 0; u < CB; ++u) {
                    dot[u] = fma(qpair.x, x[u].x, qpair.y * x[u].y);
                    w[u] = second_order && 2 * lane < D
                               ? fma(q2_s[r * D + 2 * lane], y[u].x, q2_s[r * D + 2 * lane + 1] * y[u].y)
                               : 0.0;
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1)
#pragma unroll
                    for (int u = 0; u < CB; ++u) {
                        dot[u] += __shfl_xor(dot[u], off);
                        if (second_order) w[u] += __shfl_xor(w[u], off);
                    }
#pragma unroll
                for (int u = 0; u < CB; ++u) {
                    rr[u] = s64 * dot[u];
                    if (second_order) rr[u] += fmin(0.5 * w[u], lnB);
                    if (COV) rr[u] += cov_prior(hn, j[u]);
                }
            };
            auto ambiguous = [&](int j) {
                const uint32_t x = key32(sr[j]);
                return is_cand(j) && x >= klo && x <= khi;
            };
            // mode 0: every close call is in; 1: taken-bit mask; 2: 64-bit radix threshold
            const int mode = need >= ca ? 0 : (ca <= kAmbCap ? 1 : 2);
            uint64_t t64 = 0;
            int eq_need = 0;
            if (need > 0 && mode == 1) {
                // score each close call once in fp64, then rank them (ties: lower j)
                for (int w = lane; w < NW; w += 64) tbits[w] = 0u;
                double rmine = 0.0;
                int jmine = -1;
                for (int c0 = 0; c0 < ca; c0 += CB) {     // ca <= kAmbCap here; uniform
                    int jc[CB];
                    double rc[CB];
#pragma unroll
                    for (int u = 0; u < CB; ++u) jc[u] = amb_j[min(c0 + u, ca - 1)];
                    exact_batch(jc, rc);
#pragma unroll
                    for (int u = 0; u < CB; ++u)
                        if (c0 + u < ca && lane == c0 + u) {
                            jmine = jc[u];
                            rmine = rc[u];
                            amb_r[c0 + u] = rc[u];
                        }
                }
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                if (lane < ca) {
                    int rank = 0;
                    for (int b = 0; b < ca; ++b) {
                        const double rb = amb_r[b];
                        const int jb = amb_j[b];
                        rank += (rb > rmine) || (rb == rmine && jb < jmine);
                    }
                    if (rank < need) atomicOr(&tbits[jmine >> 5], 1u << (jmine & 31));
                }
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            } else if (need > 0 && mode == 2) {
                t64 = wave_radix_select<uint64_t, 64>(
                    N, need, [&](int j) { return key64(exact(j)); }, ambiguous, hist, &eq_need);
            }
            // write ascending
            int eq_seen = 0;
#pragma unroll
            for (int t = 0; t < KPL; ++t) {
                const int j = 64 * t + lane;
                bool take = kv[t] > khi;
                bool eq = false;
                if (!take && kv[t] >= klo && kv[t] != 0u && need > 0) {
                    if (mode == 0) {
                        take = true;
                    } else if (mode == 1) {
                        take = (tbits[j >> 5] >> (j & 31)) & 1u;
                    } else {
                        const uint64_t kk = key64(exact(j));
                        take = kk > t64;
                        eq = kk == t64;
                    }
                }
                const unsigned long long eqm = __ballot(eq);
                const int eq_before = __popcll(eqm & lt_mask);
                if (eq && eq_seen + eq_before < eq_need) take = true;
                eq_seen += __popcll(eqm);
                const unsigned long long tm = __ballot(take);
                const int pos = __popcll(tm & lt_mask);
                if (take && written + pos < topk) out[written + pos] = j;
                written += __popcll(tm);
            }
        }
        for (int c = written + lane; c < topk; c += 64) out[c] = -1;
    };
    for (int r = wave; r < nq; r += NWV) {
        d2_t qp = qpre[0];
#pragma unroll
        for (int rr = 1; rr < RPW; ++rr)
            if (r == wave + rr * NWV) qp = qpre[rr];
        if (COV) qp = load_q(r);
        row_pass(r, qp);
    }
}

// General fallback for long sequences (score rows beyond the LDS): one workgroup per
// query block, fp64 scores of every candidate, radix select on 64-bit keys.
constexpr int kMaxN = 8192;

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

template <int D>
__global__ __launch_bounds__(kThreads) void route_slow_kernel(
    const double* __restrict__ qbar, const double* __restrict__ q2bar, const double* __restrict__ kbar,
    const double* __restrict__ ksig2, const double* __restrict__ hnorm, int N, double s64, int topk, int band,
    int n_sink, int second_order, int32_t* __restrict__ idx, float* __restrict__ wgate) {
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
    const double lnB = log((double)kBlock);
    if (tid < D) {
        qbar_s[tid] = qbar[(bh * N + i) * (int64_t)D + tid];
        q2_s[tid] = second_order ? q2bar[(bh * N + i) * (int64_t)D + tid] : 0.0;
    }
    __syncthreads();
    const double* kb = kbar + bh * (int64_t)N * D;
    const double* sg = second_order ? ksig2 + bh * (int64_t)N * D : nullptr;
    float* wrow = second_order ? wgate + (bh * (int64_t)N + i) * N : nullptr;
    int ncand = 0;
    for (int j = tid; j < N; j += kThreads) {
        double dot = 0.0;
        const double* kr = kb + (int64_t)j * D;
        for (int d = 0; d < D; ++d) dot = fma(qbar_s[d], kr[d], dot);
        double r = s64 * dot;
        if (second_order) {
            const double* sr = sg + (int64_t)j * D;
            double w = 0.0;
            for (int d = 0; d < D; ++d) w = fma(q2_s[d], sr[d], w);
            w *= 0.5;
            r += fmin(w, lnB);
            wrow[j] = (float)(w > lnB ? 0.0 : w);
        }
        if (hnorm) r += cov_prior(hnorm + bh * (int64_t)N, j);
        const bool cand = abs(i - j) > band && j >= n_sink;
        key_s[j] = cand ? key64(r) : 0ull;
        ncand += cand;
    }
    int dummy;
    ncand = block_scan(ncand, scan_s, &dummy);
    const int k = min(topk, ncand);
    int32_t* out = idx + (bh * (int64_t)N + i) * topk;
    if (k == 0) {
        for (int c = tid; c < topk; c += kThreads) out[c] = -1;
        return;
    }
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
    const uint64_t thr = prefix_s;
    const int need_eq = need_s;
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

hipError_t launch_route_topk(const Geom& g, const pisa_params_t* p, const StatsView* st,
                             int32_t* idx, float* wgate, hipStream_t stream) {
    const int so = p->second_order;
    if (p->topk == 0 && !so) return hipSuccess;
    const double* hn = p->cov_bias ? st->hnorm : nullptr;
    const int kc = g.N <= 64 * 8 ? 0 : (g.N <= 64 * 16 ? 1 : 2);
    const int nwv = route_waves(kc == 0 ? 8 : (kc == 1 ? 16 : kKeysPerLane));
    const size_t lds = fast_lds_bytes(g.D, g.N, so, nwv);
    if (lds + kLdsStatic <= (size_t)kLdsMax && g.N <= 64 * kKeysPerLane) {
        const dim3 block(64 * nwv);
        using Fn = void (*)(const double*, const double*, const double*, const bf16_t*, const double*,
                            const bf16_t*, const float*, const double*, int, double, int, int, int, int32_t*,
                            float*);
        static bool attr_set[2][2][2][3] = {};
#define PISA_ROUTE_ROW(DD, SO, CV) \
    {&route_fast_kernel<DD, SO, 8, CV>, &route_fast_kernel<DD, SO, 16, CV>, &route_fast_kernel<DD, SO, kKeysPerLane, CV>}
        static const Fn table[2][2][2][3] = {
            {{PISA_ROUTE_ROW(64, false, false), PISA_ROUTE_ROW(64, true, false)},
             {PISA_ROUTE_ROW(64, false, true), PISA_ROUTE_ROW(64, true, true)}},
            {{PISA_ROUTE_ROW(128, false, false), PISA_ROUTE_ROW(128, true, false)},
             {PISA_ROUTE_ROW(128, false, true), PISA_ROUTE_ROW(128, true, true)}}};
#undef PISA_ROUTE_ROW
        const int cv = hn ? 1 : 0;
        bool& set = attr_set[g.D == 128][cv][so ? 1 : 0][kc];
        const Fn fn = table[g.D == 128][cv][so ? 1 : 0][kc];
        if (!set) {   // opt in to more than 64 KB of dynamic LDS
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kLdsMax - kLdsStatic);
            if (e != hipSuccess) return e;
            set = true;
        }
        dim3 grid((g.N + kQB - 1) / kQB, (unsigned)g.BH);
        hipLaunchKernelGGL(fn, grid, block, lds, stream, st->qbar, st->q2bar, st->kbar, st->kbar_r, st->ksig2,
                           st->ksig2_r, st->knorm, hn, g.N, g.scale64, p->topk, p->band, p->n_sink, idx, wgate);
    } else {
        const dim3 grid(g.N, (unsigned)g.BH), block(kThreads);
#define PISA_ROUTE_LAUNCH(DD)                                                                      \
    hipLaunchKernelGGL(route_slow_kernel<DD>, grid, block, 0, stream, st->qbar, st->q2bar,         \
                       st->kbar, st->ksig2, hn, g.N, g.scale64, p->topk, p->band, p->n_sink, so, idx, wgate)
        if (g.D == 128) PISA_ROUTE_LAUNCH(128);
        else PISA_ROUTE_LAUNCH(64);
#undef PISA_ROUTE_LAUNCH
    }
    return hipGetLastError();
}

}  // namespace pisa
