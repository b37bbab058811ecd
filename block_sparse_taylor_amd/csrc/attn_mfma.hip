// Fused PISA forward for bf16 inputs on gfx950 bf16 MFMA (PISA, §3.4
// Algorithm 1 Phases 1-3, Eqs. 3-5 and 9-10; Piecewise-Taylor-Attention
// README for the gated second-order logit term).
//
// Work decomposition
//   One workgroup (4 wave64) per (batch*head, 64-row query block i). The
//   block's work items are its exact KV blocks (the +-band, then the routed
//   ids) followed by its virtual-token groups (64 consecutive KV blocks'
//   (kbar_j, V-hat_j / n_j) rows each). Items are dealt round-robin to the 4
//   waves; each wave keeps its own online-softmax state for all 64 query rows
//   (split-KV inside the workgroup) and the states are merged at the end, so
//   no K/V tile is shared through LDS and LDS bandwidth is spent only on V.
//
// Per item and wave (32x32x16 bf16 MFMA, fp32 accumulation):
//   S^T = K Q^T        A = K rows straight from global memory, B = Q^T from
//                      registers (loaded once); lane l holds query l%32 of
//                      query tile qt and 16 keys per key tile.
//   P   = exp2(S^T s log2e + bias - m)   bias: 0 / -inf for exact keys past
//                      T; log2 n_j + log2e w_ij, or -inf for selected blocks,
//                      for virtual tokens (a virtual token is a key with
//                      logit lam + ln n_j and value V-hat_j / n_j: mass
//                      n_j e^lam, numerator e^lam V-hat_j).
//   O^T += V^T P       A = V^T read from a per-wave LDS buffer (written
//                      transposed from registers), B = P straight from the
//                      S^T accumulator (no lane movement). O^T keeps query =
//                      lane, so the softmax rescale is a per-lane multiply.
//   The PV product of item n-1 is issued before the softmax of item n, so
//   the MFMA pipe has independent work while the VALU evaluates exponentials.
// Epilogue: every wave writes (m, l, l_tail, O^T) to LDS; wave w then merges
//   the 4 states for output dims [32w, 32w+32), adds the global first order
//   F = (l_tail / T) s (Q H) computed with bf16 MFMA on H split into
//   hi + lo bf16 parts, divides by l and stores bf16.
#include <math.h>

#include "common.h"

namespace pisa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPitch = 68;              // V^T row pitch in bf16 (64 keys + 4)
constexpr int kMaxWords = 8192 / 32;    // selection bitmask words (N <= 8192)
constexpr float kTau = 8.0f;            // stale-max tolerance of the softmax (log2 units)

template <int D>
struct Cfg {
    static constexpr int KS = D / 16;          // QK k-steps
    static constexpr int DT = D / 32;          // 32-wide output-dim tiles
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int KGP = 64 / CH;        // 4-key groups per V load pass
    static constexpr int VIT = 16 / KGP;       // V load passes
    static constexpr int VT = D * kPitch;      // bf16 elements per V^T buffer
    static constexpr int VT_BYTES = 8 * VT * 2;
    static constexpr int MERGE_BYTES = 4 * DT * 2 * 16 * 64 * 4 + 3 * 4 * 64 * 4;
    static constexpr int REGION = VT_BYTES > MERGE_BYTES ? VT_BYTES : MERGE_BYTES;
    static constexpr int QP = D + 8;           // Q row pitch in LDS (bf16)
    static constexpr int QBYTES = 64 * QP * 2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> bf16 (round to nearest even) packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ v, const bf16_t* __restrict__ kbar_c,
                      const bf16_t* __restrict__ vbar_c, const float* __restrict__ hsum,
                      const int32_t* __restrict__ idx, const float* __restrict__ wgate,
                      bf16_t* __restrict__ o, int T, int N, int total, float scale, int topk,
                      int band, int second_order, int first_order, int phase_mask) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[C::REGION + C::QBYTES];
    __shared__ uint32_t selbits[kMaxWords];
    __shared__ int nvalid_s;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int r32 = lane & 31, g = lane >> 5;

    // XCD-aware order: consecutive workgroup ids land on different XCDs; give
    // each XCD a contiguous range of (head, query block) so neighbouring query
    // blocks of one head (which route to overlapping KV blocks) share its L2.
    int L;
    {
        const int x = blockIdx.x;
        const int per = total / 8, rem = total % 8, xcd = x % 8, pos = x / 8;
        L = xcd < rem ? xcd * (per + 1) + pos : rem * (per + 1) + (xcd - rem) * per + pos;
    }
    const int64_t bh = L / N;
    const int i = L % N;

    const bool do_exact = phase_mask == 0 || (phase_mask & 1);
    const bool do_virtual = phase_mask == 0 || (phase_mask & 2);
    const bool do_first = (phase_mask == 0 || (phase_mask & 4)) && first_order;

    // ---- selection bitmask of S_i and the number of routed ids
    const int words = (N + 31) / 32;
    for (int w = tid; w < words; w += kThreads) selbits[w] = 0u;
    if (tid == 0) nvalid_s = 0;
    __syncthreads();
    const int lo = max(0, i - band), hi = min(N - 1, i + band);
    const int nb = hi - lo + 1;
    for (int c = tid; c < nb; c += kThreads) atomicOr(&selbits[(lo + c) >> 5], 1u << ((lo + c) & 31));
    const int32_t* row = topk > 0 ? idx + (bh * N + i) * (int64_t)topk : nullptr;
    int myvalid = 0;
    for (int c = tid; c < topk; c += kThreads) {
        const int j = row[c];
        if (j >= 0) {
            atomicOr(&selbits[j >> 5], 1u << (j & 31));
            ++myvalid;
        }
    }
    if (myvalid) atomicAdd(&nvalid_s, myvalid);
    __syncthreads();
    const int nvalid = nvalid_s;
    const int E = do_exact ? nb + nvalid : 0;
    const int GV = do_virtual ? (N + 63) / 64 : 0;
    const int items = E + GV;

    // ---- Q rows of the block staged once in LDS (shared by the 4 waves); the
    // Q^T operand of S^T = K Q^T is read from there: dim d = (D/2) g + 8 ks + e
    bf16_t* qs = reinterpret_cast<bf16_t*>(smem + C::REGION);
    {
        const bf16_t* qh = q + bh * (int64_t)T * D;
        for (int c = tid; c < 64 * C::CH; c += kThreads) {
            const int rr = c / C::CH, ch = c % C::CH;
            const int t = i * 64 + rr;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (t < T) u = *reinterpret_cast<const uint4*>(qh + (int64_t)t * D + 8 * ch);
            *reinterpret_cast<uint4*>(qs + rr * C::QP + 8 * ch) = u;
        }
    }
    __syncthreads();
    auto qop = [&](int qt, int ks) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(qs + (qt * 32 + r32) * C::QP + (D / 2) * g + 8 * ks));
    };

    const float c2 = scale * kLog2e;
    const float lnlast2 = log2f((float)(T - (N - 1) * 64));   // log2 n of the last block
    const float* wrow = second_order ? wgate + (bh * N + i) * (int64_t)N : nullptr;

    float m2[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f}, ltail[2] = {0.f, 0.f};
    f32x16_t acc[C::DT][2];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[dt][qt][e] = 0.f;

    bf16_t* vt_base = reinterpret_cast<bf16_t*>(smem) + wave * 2 * C::VT;

    // ---- item description
    struct Item {
        const bf16_t* ks;
        const bf16_t* vs;
        int nval;       // valid rows
        int vgroup;     // virtual group index, or -1 for an exact block
    };
    auto item_of = [&](int t) {
        Item it;
        if (t < E) {
            const int j = t < nb ? lo + t : row[t - nb];
            const int64_t off = (bh * T + (int64_t)j * 64) * D;
            it.ks = k + off;
            it.vs = v + off;
            it.nval = min(64, T - j * 64);
            it.vgroup = -1;
        } else {
            const int gi = t - E;
            const int64_t off = (bh * N + (int64_t)gi * 64) * D;
            it.ks = kbar_c + off;
            it.vs = vbar_c + off;
            it.nval = min(64, N - gi * 64);
            it.vgroup = gi;
        }
        return it;
    };

    uint4 kreg[2][C::KS];
    uint4 vreg[C::VIT][4];
    // Rows past the item's valid count are read from its last valid row and
    // zeroed, so every load is unconditional (no divergent branches).
    auto load_k = [&](const Item& it) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int rr = kt * 32 + r32;
            const bool ok = rr < it.nval;
            const bf16_t* src = it.ks + (ok ? rr : it.nval - 1) * D + (D / 2) * g;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                uint4 u = *reinterpret_cast<const uint4*>(src + 8 * ks);
                if (!ok) u = make_uint4(0, 0, 0, 0);
                kreg[kt][ks] = u;
            }
        }
    };
    const int vc = lane % C::CH, vkg0 = lane / C::CH;
    auto load_v = [&](const Item& it) {
#pragma unroll
        for (int p = 0; p < C::VIT; ++p)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = 4 * (vkg0 + C::KGP * p) + r;
                const bool ok = key < it.nval;
                uint4 u = *reinterpret_cast<const uint4*>(it.vs + (ok ? key : it.nval - 1) * D + 8 * vc);
                if (!ok) u = make_uint4(0, 0, 0, 0);
                vreg[p][r] = u;
            }
    };
    // V rows (registers) -> V^T buffer: 4 keys x 8 dims per (pass), 4x4 bf16 transposes
    auto store_vt = [&](bf16_t* buf) {
#pragma unroll
        for (int p = 0; p < C::VIT; ++p) {
            const int kg = vkg0 + C::KGP * p;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t a0 = (&vreg[p][0].x)[w], a1 = (&vreg[p][1].x)[w];
                const uint32_t a2 = (&vreg[p][2].x)[w], a3 = (&vreg[p][3].x)[w];
                const uint2 lo2 = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x05040100u),
                                             __builtin_amdgcn_perm(a3, a2, 0x05040100u));
                const uint2 hi2 = make_uint2(__builtin_amdgcn_perm(a1, a0, 0x07060302u),
                                             __builtin_amdgcn_perm(a3, a2, 0x07060302u));
                const int d = 8 * vc + 2 * w;
                *reinterpret_cast<uint2*>(buf + d * kPitch + 4 * kg) = lo2;
                *reinterpret_cast<uint2*>(buf + (d + 1) * kPitch + 4 * kg) = hi2;
            }
        }
    };

    bf16x8_t pp[2][2][2];   // [kt][half][qt] P operands of the previous item
    auto pv = [&](const bf16_t* buf) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const bf16_t* vrow = buf + (dt * 32 + r32) * kPitch + 4 * g;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int base = kt * 32 + half * 16;
                    const uint2 a = *reinterpret_cast<const uint2*>(vrow + base);
                    const uint2 b = *reinterpret_cast<const uint2*>(vrow + base + 8);
                    const bf16x8_t av = as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pp[kt][half][qt], acc[dt][qt], 0, 0, 0);
                }
        }
    };

    int t = wave;
    bool has_prev = false;
    int parity = 0;
    Item cur;
    if (t < items) {
        cur = item_of(t);
        load_k(cur);
    }
    for (; t < items; t += 4) {
        // this item's V^T into its buffer (the buffer PV read two items ago)
        load_v(cur);
        // S^T = K Q^T
        f32x16_t s[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kt][qt][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks)
                    s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][ks]), qop(qt, ks), s[kt][qt], 0, 0, 0);
            }
        // this item's V^T into its buffer (the one PV read two items ago)
        store_vt(vt_base + parity * C::VT);
        const bool has_next = t + 4 < items;
        Item nxt = cur;
        // O^T += V^T P of the previous item (independent of this item's softmax)
        if (has_prev) pv(vt_base + (parity ^ 1) * C::VT);
        if (has_next) {
            nxt = item_of(t + 4);
            load_k(nxt);
        }

        // softmax of this item. The reference max m2 only moves when a tile
        // exceeds it by more than kTau (log2 units); otherwise P <= 2^kTau is
        // taken against the stale max and the accumulator is not rescaled.
        const bool virt = cur.vgroup >= 0;
        const bool full = !virt && cur.nval == 64;
        float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int run = 0; run < 4; ++run) {
                // keys kt*32 + 8 run + 4 g + (0..3) of this lane
                const int key0 = kt * 32 + 8 * run + 4 * g;
                float b[4] = {0.f, 0.f, 0.f, 0.f};
                if (!full) {
                    if (!virt) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) b[e] = key0 + e < cur.nval ? 0.f : -INFINITY;
                    } else {
                        const int j0 = cur.vgroup * 64 + key0;
                        const uint32_t bits = j0 < N ? (selbits[j0 >> 5] >> (j0 & 31)) : 0xFu;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int j = j0 + e;
                            float bb = j == N - 1 ? lnlast2 : 6.0f;   // log2 n_j
                            if (second_order) bb += kLog2e * wrow[min(j, N - 1)];
                            b[e] = (j >= N || ((bits >> e) & 1u)) ? -INFINITY : bb;
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) {
                        const float z = fmaf(s[kt][qt][4 * run + e], c2, b[e]);
                        s[kt][qt][4 * run + e] = z;
                        mx[qt] = fmaxf(mx[qt], z);
                    }
            }
        bool need = false;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            mx[qt] = fmaxf(mx[qt], __shfl_xor(mx[qt], 32));
            need |= mx[qt] > m2[qt] + kTau;
        }
        if (__any(need)) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                const float mnew = fmaxf(m2[qt], mx[qt]);
                const float alpha = fast_exp2(m2[qt] - (mnew == -INFINITY ? 0.f : mnew));
                m2[qt] = mnew;
                lsum[qt] *= alpha;
                ltail[qt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[dt][qt][e] *= alpha;
            }
        }
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float muse = m2[qt] == -INFINITY ? 0.f : m2[qt];
            float rs = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float pe = fast_exp2(s[kt][qt][e] - muse);
                    s[kt][qt][e] = pe;
                    rs += pe;
                }
            lsum[qt] += rs;
            if (virt) ltail[qt] += rs;
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    uint4 u;
                    u.x = pack_bf16x2(s[kt][qt][8 * half + 0], s[kt][qt][8 * half + 1]);
                    u.y = pack_bf16x2(s[kt][qt][8 * half + 2], s[kt][qt][8 * half + 3]);
                    u.z = pack_bf16x2(s[kt][qt][8 * half + 4], s[kt][qt][8 * half + 5]);
                    u.w = pack_bf16x2(s[kt][qt][8 * half + 6], s[kt][qt][8 * half + 7]);
                    pp[kt][half][qt] = as_bf16x8(u);
                }

        cur = nxt;
        has_prev = true;
        parity ^= 1;
    }
    if (has_prev) pv(vt_base + (parity ^ 1) * C::VT);

    // ---- merge the four wave states and finish (Phase 3)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        lsum[qt] += __shfl_xor(lsum[qt], 32);
        ltail[qt] += __shfl_xor(ltail[qt], 32);
    }
    __syncthreads();   // every wave is done with its V^T buffers
    float* mo = reinterpret_cast<float*>(smem);
    float* ms = mo + 4 * C::DT * 2 * 16 * 64;
    float* ls = ms + 4 * 64;
    float* lts = ls + 4 * 64;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mo[(((wave * C::DT + dt) * 2 + qt) * 16 + e) * 64 + lane] = acc[dt][qt][e];
    if (g == 0) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            ms[wave * 64 + qt * 32 + r32] = m2[qt];
            ls[wave * 64 + qt * 32 + r32] = lsum[qt];
            lts[wave * 64 + qt * 32 + r32] = ltail[qt];
        }
    }
    __syncthreads();
    if (wave >= C::DT) return;
    const int dt = wave;

    // G^T = H^T Q^T for output dims [32 dt, 32 dt + 32): A = H^T split hi + lo
    f32x16_t gacc[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int e = 0; e < 16; ++e) gacc[qt][e] = 0.f;
    if (do_first) {
        const float* H = hsum + bh * (int64_t)D * D;
        const int ecol = dt * 32 + r32;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            bf16x8_t ah, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = (D / 2) * g + 8 * ks + e;
                const float h = H[d * D + ecol];
                const bf16_t hb = f32_to_bf16(h);
                ah[e] = __builtin_bit_cast(__bf16, hb);
                al[e] = __builtin_bit_cast(__bf16, f32_to_bf16(h - bf16_to_f32(hb)));
            }
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                gacc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qop(qt, ks), gacc[qt], 0, 0, 0);
                gacc[qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qop(qt, ks), gacc[qt], 0, 0, 0);
            }
        }
    }
    bf16_t* oh = o + bh * (int64_t)T * D;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int qi = qt * 32 + r32;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, ms[w * 64 + qi]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float f[4], Lsum = 0.f, LT = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            f[w] = fast_exp2(ms[w * 64 + qi] - Mu);
            Lsum = fmaf(f[w], ls[w * 64 + qi], Lsum);
            LT = fmaf(f[w], lts[w * 64 + qi], LT);
        }
        const float cF = do_first ? scale * LT / (float)T : 0.f;
        const float inv = 1.f / Lsum;
        float out[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float a = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) a = fmaf(f[w], mo[(((w * C::DT + dt) * 2 + qt) * 16 + e) * 64 + lane], a);
            out[e] = (a + cF * gacc[qt][e]) * inv;
        }
        const int trow = i * 64 + qi;
        if (trow < T) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = dt * 32 + 8 * a4 + 4 * g;
                uint2 u;
                u.x = pack_bf16x2(out[4 * a4 + 0], out[4 * a4 + 1]);
                u.y = pack_bf16x2(out[4 * a4 + 2], out[4 * a4 + 3]);
                *reinterpret_cast<uint2*>(oh + (int64_t)trow * D + d0) = u;
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_fwd_mfma(const Geom& g, const pisa_params_t* p, const void* q, const void* k,
                                const void* v, const pisa_stats_t* st, const int32_t* idx,
                                const float* wgate, void* o, hipStream_t stream) {
    const int64_t total64 = g.BH * (int64_t)g.N;
    if (total64 > (int64_t)0x7fffffff) return hipErrorInvalidValue;
    const int total = (int)total64;
    dim3 grid(total), block(kThreads);
#define PISA_MFMA_LAUNCH(DD)                                                                        \
    hipLaunchKernelGGL((attn_mfma_kernel<DD>), grid, block, 0, stream,                              \
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),                \
                       static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(st->kbar_c),       \
                       static_cast<const bf16_t*>(st->vbar_c), st->hsum, idx, wgate,                \
                       static_cast<bf16_t*>(o), g.T, g.N, total, g.scale, p->topk, p->band,         \
                       p->second_order, p->first_order, p->phase_mask)
    if (g.D == 128) PISA_MFMA_LAUNCH(128);
    else PISA_MFMA_LAUNCH(64);
#undef PISA_MFMA_LAUNCH
    return hipGetLastError();
}

}  // namespace pisa
