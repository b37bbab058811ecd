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
//   (split-KV inside the workgroup) and the states are merged at the end.
//
// Per item and wave (32x32x16 bf16 MFMA, fp32 accumulation):
//   S^T = K Q^T     A = K rows by buffer loads straight into registers (the
//                   buffer descriptor's record count zero-fills rows past the
//                   item's end); B = Q^T from an LDS copy shared by the waves.
//                   Lane l then holds query l%32 of query tile qt, 16 keys
//                   per key tile.
//   P = exp2(S^T s log2e + bias - m)   bias: -inf for keys past T; for
//                   virtual tokens log2 n_j + log2e w_ij, or -inf for
//                   selected blocks (a virtual token is a key with logit
//                   lam + ln n_j and value V-hat_j / n_j).
//   O^T += V^T P    B = P straight from the S^T accumulator (no lane
//                   movement); A = V^T read with the gfx950 LDS transpose
//                   read from a row-major V tile (rows XOR-swizzled by
//                   row % 4 in 8-byte units, so 16-byte row writes and the
//                   transposed reads are both bank-conflict free). O^T keeps
//                   query = lane, so any rescale is a per-lane multiply.
//   The reference max only moves when a tile exceeds it by more than kTau
//   (log2 units); otherwise P <= 2^kTau is taken against the stale max and
//   the accumulator is left alone. The PV product of item n-1 is issued
//   before the softmax of item n.
// Epilogue: every wave writes (m, l, l_tail, O^T) to LDS; wave w merges the
//   4 states for output dims [32w, 32w+32), adds the global first order
//   F = (l_tail / T) s (Q H) (bf16 MFMA on H split into hi + lo parts),
//   divides by l and stores bf16.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace pisa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxWords = 8192 / 32;    // selection bitmask words (N <= 8192)
constexpr float kTau = 64.0f;           // headroom of the fixed softmax reference (log2 units)
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // gfx9 raw buffer descriptor, dword 3

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct Cfg {
    static constexpr int KS = D / 16;          // QK k-steps
    static constexpr int DT = D / 32;          // 32-wide output-dim tiles
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int VL = CH;              // V DMA instructions per item (64 rows * CH / 64)
    static constexpr int RB = 2 * D;           // row bytes
    static constexpr int VBUF = 64 * RB;       // bytes of one V tile
    static constexpr int QP = D + 8;           // Q row pitch in LDS (bf16)
    // the merge of the wave states reuses the V tiles: two waves' O^T per parity array
    static_assert(2 * DT * 2 * 16 * 64 * 4 == 4 * VBUF, "merge layout");
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp32 -> bf16 (round to nearest even) packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer descriptor of a wave-uniform range. The fields are passed through
// readfirstlane so the descriptor stays in SGPRs even where the compiler
// cannot prove uniformity (a VGPR descriptor becomes a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                             (int)kRsrcWord3);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes M0 base +
// 16 l (the LDS address is wave-uniform). The host pass of this compiler
// drops any kernel whose body names this builtin, so only the device pass
// sees it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff,
                                      uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             (int)voff, (int)soff, 0, 0);
#endif
}

__device__ __forceinline__ uint2 lds_tr16(const unsigned char* p) {
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_mfma_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                      const bf16_t* __restrict__ v, const bf16_t* __restrict__ kbar_c,
                      const bf16_t* __restrict__ vbar_c, const float* __restrict__ hsum,
                      const int32_t* __restrict__ idx, const float* __restrict__ wgate,
                      bf16_t* __restrict__ o, int T, int N, int total, float scale, int topk,
                      int band, int second_order, int first_order, int phase_mask) {
    using C = Cfg<D>;
    // V tiles of the two pipeline parities live in separate arrays, so that the
    // compiler can tell the asynchronous buffer->LDS writes into one parity from
    // reads of the other (and of the Q tile) and waits only where data is needed.
    __shared__ __attribute__((aligned(16))) unsigned char vb0[4 * C::VBUF];
    __shared__ __attribute__((aligned(16))) unsigned char vb1[4 * C::VBUF];
    __shared__ __attribute__((aligned(16))) bf16_t qs[64 * C::QP];
    __shared__ float mstat[3 * 4 * 64];
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

    // ---- Q rows of the block staged once in LDS (shared by the 4 waves); the
    // Q^T operand of S^T = K Q^T is read from there: dim d = (D/2) g + 8 ks + e
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
    const int nvalid = __builtin_amdgcn_readfirstlane(nvalid_s);   // LDS value, uniform: keep item data in SGPRs
    const int E = do_exact ? nb + nvalid : 0;
    const int GV = do_virtual ? (N + 63) / 64 : 0;
    const int items = E + GV;
    // per-lane element offset of the Q^T operand; each step launders it so the
    // compiler re-reads Q from LDS per item instead of pinning its 16 operands
    // (64 VGPRs) in registers for the whole loop
    const int qlane = r32 * C::QP + (D / 2) * g;
    auto qop_at = [&](int qb, int qt, int ks) {
        return as_bf16x8(*reinterpret_cast<const uint4*>(qs + qb + qt * 32 * C::QP + 8 * ks));
    };
    auto qop = [&](int qt, int ks) { return qop_at(qlane, qt, ks); };

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


    // ---- item description (wave-uniform: lives in SGPRs)
    struct Item {
        const bf16_t* ks;
        const bf16_t* vs;
        int nval;       // valid rows
        int vgroup;     // virtual group index, or -1 for an exact block
    };
    typedef __attribute__((address_space(4))) const int32_t cint32_t;
    cint32_t* crow = (cint32_t*)(uintptr_t)row;   // uniform index: scalar loads
    auto item_of = [&](int t) {
        Item it;
        if (t < E) {
            const int j = t < nb ? lo + t : crow[t - nb];
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

    // Per-lane byte offsets (constant over items)
    const uint32_t koff = (uint32_t)(r32 * C::RB + D * g);              // K operand: row r32, dims (D/2) g..
    // V tile: buffer -> LDS DMA, 1 KB per instruction: lane l fills LDS slot l,
    // i.e. row RPI n + l / CH, 16-byte position l % CH. That position holds
    // the row's chunk (l % CH) ^ 2 (row % 4) (the swizzle the transposed
    // reads expect), so the lane loads that chunk. RPI = 64 / CH rows per
    // instruction is a multiple of 4, so row % 4 = (l / CH) % 4 for every n.
    constexpr int RPI = 64 / C::CH;
    const int vrow0 = lane / C::CH;
    const uint32_t voff = (uint32_t)(vrow0 * C::RB + 16 * ((lane % C::CH) ^ (2 * (vrow0 & 3))));

    uint4 kreg[2][C::KS];
    auto load_k = [&](const Item& it) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(it.ks, (uint32_t)(it.nval * C::RB));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) kreg[kt][ks] = bload16(r, koff + kt * 32 * C::RB + 16 * ks);
    };
    // Rows past the item's end are zero-filled by the descriptor's range check.
    auto dma_v = [&](const Item& it, unsigned char* buf) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(it.vs, (uint32_t)(it.nval * C::RB));
#pragma unroll
        for (int n = 0; n < C::VL; ++n)
            dma16(r, buf + n * RPI * C::RB, voff, n * RPI * C::RB);
    };

    // Transposed-read addresses (lane-constant part): in each 16-lane group,
    // lane a + 4e fetches row base + 4g + e, dims C0 + 4a (8 bytes); the read
    // hands lane 4a + b element b of the fetches of lanes a, a+4, a+8, a+12.
    const int trG = lane >> 4, tri = lane & 15, tra = tri & 3, tre = tri >> 2;
    const uint32_t trow = (uint32_t)((4 * g + tre) * C::RB);
    auto tr_off = [&](int dt) {   // byte offset within a row of this lane's 8-byte chunk
        const int c8 = (dt * 32 + 16 * (trG & 1) + 4 * tra) >> 2;
        return (uint32_t)(8 * (c8 ^ (4 * tre)));
    };

    bf16x8_t pp[2][2][2];   // [kt][half][qt] P operands of the previous item
    auto pv = [&](const unsigned char* buf) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
            const unsigned char* base = buf + trow + tr_off(dt);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int r0 = kt * 32 + half * 16;
                    const uint2 a = lds_tr16(base + r0 * C::RB);
                    const uint2 b = lds_tr16(base + (r0 + 8) * C::RB);
                    const bf16x8_t av = as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pp[kt][half][qt], acc[dt][qt], 0, 0, 0);
                }
        }
    };

    // Pipeline per wave: item n's K sits in registers (loaded during item n-1)
    // and its V tile in LDS buffer n % 2 (DMA issued during item n-1, right
    // after PV of item n-2 released that buffer).
    //
    // Softmax reference: the accumulator is never rescaled. A query's
    // reference m2 is the first finite tile max it sees (its accumulator is
    // still zero then); later tiles are taken against it, P = 2^(z - m2) <=
    // 2^kTau. If a tile ever exceeds its reference by more than kTau, the wave
    // raises the reference and restarts its items from zero (each restart
    // raises some reference by more than kTau, so restarts are finite).
    // One pipeline step for the wave's current item `cur` (its K already in
    // registers), with the V tiles of parity PAR: DMA cur's V into this
    // parity's tile (its last reader, the PV of the item before the previous
    // one, has finished), S^T = K Q^T, K loads of the next item, PV of the
    // previous item (its V arrived during the previous step), softmax of cur.
    int t = 0;
    bool has_prev = false;
    Item cur;
    auto step = [&](auto par) -> bool {
        constexpr int PAR = decltype(par)::value;
        unsigned char* vcur = (PAR == 0 ? vb0 : vb1) + wave * C::VBUF;
        const unsigned char* vprev = (PAR == 0 ? vb1 : vb0) + wave * C::VBUF;
        dma_v(cur, vcur);
        // S^T = K Q^T
        int qb = qlane;
        asm volatile("" : "+v"(qb));
        f32x16_t s[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
                for (int e = 0; e < 16; ++e) s[kt][qt][e] = 0.f;
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks)
                    s[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kreg[kt][ks]), qop_at(qb, qt, ks), s[kt][qt], 0, 0, 0);
            }
        const bool has_next = t + 4 < items;
        Item nxt = cur;
        if (has_next) {
            nxt = item_of(t + 4);
            load_k(nxt);
        }
        // O^T += V^T P of the previous item (independent of this item's softmax)
        if (has_prev) pv(vprev);

        // ---- softmax of this item
        const bool virt = cur.vgroup >= 0;
        const bool plain = !virt && cur.nval == 64;   // no masking, no bias
        float mx[2] = {-INFINITY, -INFINITY};
        if (plain) {
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                float a = s[0][qt][0];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) a = fmaxf(a, s[kt][qt][e]);
                mx[qt] = a * c2;
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int run = 0; run < 4; ++run) {
                    // keys kt*32 + 8 run + 4 g + (0..3) of this lane
                    const int key0 = kt * 32 + 8 * run + 4 * g;
                    float b[4];
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
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int qt = 0; qt < 2; ++qt) {
                            const float z = fmaf(s[kt][qt][4 * run + e], c2, b[e]);
                            s[kt][qt][4 * run + e] = z;
                            mx[qt] = fmaxf(mx[qt], z);
                        }
                }
        }
        bool need = false;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            {   // lanes l and l ^ 32 hold the same query: swap halves and combine
                const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx[qt]),
                                                                 __builtin_bit_cast(uint32_t, mx[qt]), false, false);
                mx[qt] = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
            }
            if (m2[qt] == -INFINITY) m2[qt] = mx[qt];   // first finite max: accumulator still zero
            need |= mx[qt] > m2[qt] + kTau;
        }
        if (__builtin_amdgcn_ballot_w64(need) != 0) {   // ballot is wave-uniform
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) m2[qt] = fmaxf(m2[qt], mx[qt]);
            return true;
        }
        typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
        const bf16x2v_t ones = {(__bf16)1.0f, (__bf16)1.0f};
        const float cm = plain ? c2 : 1.0f;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const float muse = m2[qt] == -INFINITY ? 0.f : m2[qt];
            float rs = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    uint32_t w[4];
#pragma unroll
                    for (int h2 = 0; h2 < 4; ++h2) {
                        const float p0 = fast_exp2(fmaf(s[kt][qt][8 * half + 2 * h2], cm, -muse));
                        const float p1 = fast_exp2(fmaf(s[kt][qt][8 * half + 2 * h2 + 1], cm, -muse));
                        w[h2] = pack_bf16x2(p0, p1);
                        // row sum of the rounded weights (the ones PV uses)
                        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[h2]), ones, rs, false);
                    }
                    pp[kt][half][qt] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
                }
            lsum[qt] += rs;
            if (virt) ltail[qt] += rs;
        }
        cur = nxt;
        has_prev = true;
        return false;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    int last_par = 0;
    for (;;) {
        t = wave;
        has_prev = false;
        last_par = 0;
        bool restart = false;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[dt][qt][e] = 0.f;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            lsum[qt] = 0.f;
            ltail[qt] = 0.f;
        }
        if (t < items) {
            cur = item_of(t);
            load_k(cur);
        }
        while (t < items) {
            if (step(I0{})) {
                restart = true;
                break;
            }
            last_par = 0;
            t += 4;
            if (t >= items) break;
            if (step(I1{})) {
                restart = true;
                break;
            }
            last_par = 1;
            t += 4;
        }
        if (!restart) break;
        __builtin_amdgcn_s_waitcnt(0);   // drain the abandoned prefetches before reusing the tiles
    }
    if (has_prev) pv((last_par == 0 ? vb0 : vb1) + wave * C::VBUF);

    // ---- merge the four wave states and finish (Phase 3)
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        lsum[qt] += __shfl_xor(lsum[qt], 32);
        ltail[qt] += __shfl_xor(ltail[qt], 32);
    }
    __syncthreads();   // every wave is done with its V tiles
    // wave w's O^T goes to the tile array of parity w / 2 (two waves per array)
    auto mo_of = [&](int w) {
        return reinterpret_cast<float*>(w < 2 ? vb0 : vb1) + (w & 1) * (C::DT * 2 * 16 * 64);
    };
    float* ms = mstat;
    float* ls = mstat + 4 * 64;
    float* lts = mstat + 8 * 64;
    {
        float* mo = mo_of(wave);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
#pragma unroll
                for (int e = 0; e < 16; ++e) mo[((dt * 2 + qt) * 16 + e) * 64 + lane] = acc[dt][qt][e];
    }
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
            for (int w = 0; w < 4; ++w) a = fmaf(f[w], mo_of(w)[((dt * 2 + qt) * 16 + e) * 64 + lane], a);
            out[e] = (a + cF * gacc[qt][e]) * inv;
        }
        const int trow_o = i * 64 + qi;
        if (trow_o < T) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = dt * 32 + 8 * a4 + 4 * g;
                uint2 u;
                u.x = pack_bf16x2(out[4 * a4 + 0], out[4 * a4 + 1]);
                u.y = pack_bf16x2(out[4 * a4 + 2], out[4 * a4 + 3]);
                *reinterpret_cast<uint2*>(oh + (int64_t)trow_o * D + d0) = u;
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
