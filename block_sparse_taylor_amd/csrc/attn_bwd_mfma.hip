// Exact-pair parts of the backward on the matrix cores (bf16 inputs): the
// block-sparse softmax-attention gradient of the exact branch (PISA §3.2
// Eqs. 3-4 differentiated; Piecewise-Taylor-Attention README, trainable
// regime), computed in 64 x 64 (query block, KV block) tiles with bf16 MFMA
// 32x32x16 and fp32 accumulation.
//
//   exact_stats: per query row, max m2 and sum l of 2^(z log2e - m2) over
//                the exact keys (S^T = K Q^T), merged later with the virtual
//                tokens into lse;
//   dq_exact:    dQ^T += K^T dS^T with dS^T = P^T (dP^T - delta),
//                P^T = exp(S^T - lse), dP^T = V dO^T, added to the partial dq
//                of the virtual tokens and written in bf16;
//   dkdv_exact:  S = Q K^T and dP = dO V^T with the keys on the lanes, then
//                dV^T += dO^T P and dK^T += Q^T dS; fp32 partials for the
//                chain kernel.
// A product over queries (or keys) takes its B operand straight from an
// accumulator (the lane keeps its key, or query; the k-slots hold the
// accumulator's 8 rows of a 16-row half, 4g + (0..3) and 8 + 4g + (0..3)),
// and its A operand from the gfx950 LDS transpose read of a row-major tile
// whose 16-byte chunks are XOR-swizzled by row % 4 (the read then hands
// every lane the same 8 rows). dS and P are split into bf16 hi + lo parts
// (two MFMAs each), so the cancelling sums dq = sum dS k, dk = sum dS q and
// dv = sum P dout keep about 16 bits of every term.
// Work per workgroup (4 waves): one 64-row block against a stream of 64-row
// tiles; wave w takes the 32 x 32 sub-tile (w >> 1, w & 1) of each product
// and the two waves sharing an output tile add their partials at the end.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace pisa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct BC {
    static_assert(2 * (D / 32) * 16 * 64 * 4 == 2 * 64 * 2 * D, "the partial exchange fills the two tiles");
    static constexpr int KS = D / 16;          // k-steps over the head dim
    static constexpr int DT = D / 32;          // 32-wide head-dim tiles
    static constexpr int CH = D / 8;           // 16-byte chunks per row
    static constexpr int RB = 2 * D;           // row bytes
    static constexpr int TILE = 64 * RB;       // bytes of one 64-row tile
    static constexpr int LPT = 64 * CH / kThreads;   // 16-byte loads per thread per tile
    static constexpr int SWM = CH / 2 - 1;           // low row bits of the swizzle (below)
};

// Chunk c of row r of a staged tile sits at 16-byte position c ^ swz(r). For
// D = 128 (16 chunks per row), swz(r) = 2 (r & 7) | ((r >> 3) & 1): the 16
// consecutive rows that one row-format read serves (16 lanes at a time, one
// chunk each) land on 16 distinct positions, and a transposed read, which
// covers 8 rows starting at a multiple of 8, sees bit 0 constant, so its
// lanes keep the distinct positions of 2 (r & 7). (Measured on gfx950 with a
// standalone pattern benchmark: 2 (r & 7) alone costs row reads a two-way
// bank conflict; r & 15 makes the transposed reads conflict.) D = 64 keeps
// swz(r) = 2 (r & 3).
template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? ((2 * (r & 7)) | ((r >> 3) & 1)) : 2 * (r & BC<D>::SWM);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint2 lds_tr16(const unsigned char* p) {
    typedef __attribute__((address_space(3))) v4i16_t lds_v4i16;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p));
}

// 2^x by the hardware instruction (no denormal handling: every argument here
// is a logit minus the row's log-normaliser, so <= ~0, or -inf).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }


__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t zero16() {
    f32x16_t z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
}

// A 64-row tile (rows >= nval zero) from global memory into registers, then
// into LDS with chunk c of row r at 16-byte position c ^ swz(r).
template <int D>
__device__ __forceinline__ void tile_load(uint4 (&r)[BC<D>::LPT], const bf16_t* src, int nval, int tid) {
#pragma unroll
    for (int n = 0; n < BC<D>::LPT; ++n) {
        const int c = tid + kThreads * n;
        const int row = c / BC<D>::CH, ch = c % BC<D>::CH;
        r[n] = row < nval ? *reinterpret_cast<const uint4*>(src + (int64_t)row * D + 8 * ch) : make_uint4(0, 0, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void tile_store(unsigned char* lds, const uint4 (&r)[BC<D>::LPT], int tid) {
#pragma unroll
    for (int n = 0; n < BC<D>::LPT; ++n) {
        const int c = tid + kThreads * n;
        const int row = c / BC<D>::CH, ch = c % BC<D>::CH;
        *reinterpret_cast<uint4*>(lds + row * BC<D>::RB + 16 * (ch ^ swz<D>(row))) = r[n];
    }
}

// Row-format operand: row rr of a swizzled tile, head dims 16 ks + 8 g + (0..7).
template <int D>
__device__ __forceinline__ bf16x8_t row_op(const unsigned char* lds, int rr, int ks, int g) {
    return as_bf16x8(*reinterpret_cast<const uint4*>(lds + rr * BC<D>::RB + 16 * ((2 * ks + g) ^ swz<D>(rr))));
}

// Row-format operand straight from global memory (row t of a [T, D] matrix; zero past T).
template <int D>
__device__ __forceinline__ void rows_from_global(uint4 (&r)[BC<D>::KS], const bf16_t* base, int t, int T, int g) {
#pragma unroll
    for (int ks = 0; ks < BC<D>::KS; ++ks)
        r[ks] = t < T ? *reinterpret_cast<const uint4*>(base + (int64_t)t * D + 16 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
}

// Transposed-read addressing (lane-constant part) of a swizzled tile: the
// A operand "rows = head dims of tile dt, k = tile rows r0 + 4g + (0..3) and
// r0 + 8 + 4g + (0..3)". A lane reads row R = r0 (+ 8) + 4g + tre with r0 a
// multiple of 8, so R & SWM = (4g + tre) & SWM does not depend on r0; the
// remaining swizzle bit of D = 128, (R >> 3) & 1, is that of r0 (and of r0 +
// 8 for the second read) and enters as 16 bytes in tr_op.
struct TrAddr {
    uint32_t trow;
    int trG, tra, sw;
    __device__ TrAddr(int lane, int rb, int swm) {
        const int g = lane >> 5, tri = lane & 15;
        const int tre = tri >> 2;
        trG = lane >> 4;
        tra = tri & 3;
        sw = (4 * g + tre) & swm;
        trow = (uint32_t)((4 * g + tre) * rb);
    }
    __device__ uint32_t off(int dt) const {
        const int c8 = (dt * 32 + 16 * (trG & 1) + 4 * tra) >> 2;   // 8-byte unit
        return (uint32_t)(8 * (c8 ^ (4 * sw)));
    }
};

template <int D>
__device__ __forceinline__ bf16x8_t tr_op(const unsigned char* lds, const TrAddr& ta, int dt, int r0) {
    const uint32_t o = ta.off(dt);
    const uint32_t oa = D == 128 ? o ^ (uint32_t)(16 * ((r0 >> 3) & 1)) : o;
    const uint32_t ob = D == 128 ? o ^ (uint32_t)(16 * (((r0 + 8) >> 3) & 1)) : o;
    const uint2 a = lds_tr16(lds + ta.trow + oa + r0 * BC<D>::RB);
    const uint2 b = lds_tr16(lds + ta.trow + ob + (r0 + 8) * BC<D>::RB);
    return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}

// Registers 8 h .. 8 h + 7 of an accumulator as a bf16 B operand, and the
// remainder (x - bf16(x)) as a second one.
__device__ __forceinline__ void split_op(const f32x16_t& x, int h, bf16x8_t& hi, bf16x8_t& lo) {
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const float a = x[8 * h + 2 * p], b = x[8 * h + 2 * p + 1];
        wh[p] = pack_bf16x2(a, b);
        wl[p] = pack_bf16x2(a - bf16_lo(wh[p]), b - bf16_hi(wh[p]));
    }
    hi = as_bf16x8(make_uint4(wh[0], wh[1], wh[2], wh[3]));
    lo = as_bf16x8(make_uint4(wl[0], wl[1], wl[2], wl[3]));
}

// accumulator register r <-> tile row 8 (r / 4) + 4 g + r % 4
__device__ __forceinline__ int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// ---------------------------------------------------------------- prep
// bf16 hi + lo planes (x = hi + lo to ~16 bits) of kbar and V-hat per block
// (blockIdx.x < N) and of H per head (blockIdx.x == N): operands of the
// virtual-token and first-order products.
__device__ __forceinline__ void split_store(float x, bf16_t* hi, bf16_t* lo) {
    const bf16_t h = f32_to_bf16(x);
    *hi = h;
    *lo = f32_to_bf16(x - bf16_to_f32(h));
}

__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const double* __restrict__ kbar,
                                                            const float* __restrict__ vsum,
                                                            const float* __restrict__ hsum, bf16_t* __restrict__ kbh,
                                                            bf16_t* __restrict__ kbl, bf16_t* __restrict__ vhh,
                                                            bf16_t* __restrict__ vhl, bf16_t* __restrict__ hh,
                                                            bf16_t* __restrict__ hl, int N, int D) {
    const int64_t bh = blockIdx.y;
    if ((int)blockIdx.x < N) {
        const int64_t a0 = (bh * N + blockIdx.x) * (int64_t)D;
        for (int d = threadIdx.x; d < D; d += kThreads) {
            split_store((float)kbar[a0 + d], kbh + a0 + d, kbl + a0 + d);
            split_store(vsum[a0 + d], vhh + a0 + d, vhl + a0 + d);
        }
    } else {
        const int64_t a0 = bh * (int64_t)D * D;
        for (int e = threadIdx.x; e < D * D; e += kThreads) split_store(hsum[a0 + e], hh + a0 + e, hl + a0 + e);
    }
}

// Virtual-token logit bias of block j for query block i (log2 units), or
// -inf where j is not a virtual token of i (exact, or past N).
// Buffer descriptor of a wave-uniform range of `bytes`: loads past it read
// zero, so a tile of fewer than 64 rows loads without per-row branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes the
// wave-uniform LDS address + 16 l. The host pass of this compiler drops any
// kernel whose body names this builtin, so only the device pass sees it.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, 0, 0, 0);
#endif
}

// A 64-row tile into LDS by buffer->LDS DMA, in the staged layout (chunk c of
// row r at 16-byte position c ^ swz(r)): 1 KB instruction n fills LDS bytes
// [1024 n, 1024 n + 1024), i.e. rows RPI n .. RPI n + RPI - 1, so lane l,
// landing on row RPI n + l / CH at position l % CH, loads that row's chunk
// (l % CH) ^ swz(row). Each of the 4 waves issues a quarter of the
// instructions; rows past the descriptor's range read zero.
template <int D>
__device__ __forceinline__ void tile_dma(unsigned char* lds, __amdgpu_buffer_rsrc_t r, int wave, int lane) {
    constexpr int NI = BC<D>::TILE / 1024, RPI = 1024 / BC<D>::RB;
    static_assert(NI % 4 == 0 && kThreads == 256, "four waves share a tile's DMA instructions");
#pragma unroll
    for (int m = 0; m < NI / 4; ++m) {
        const int n = wave * (NI / 4) + m;
        const int row = RPI * n + lane / BC<D>::CH, pos = lane % BC<D>::CH;
        dma16(r, lds + 1024 * n, (uint32_t)(row * BC<D>::RB + 16 * (pos ^ swz<D>(row))));
    }
}

// The staged tile of tile_dma, issued from inline asm: the compiler does not
// count these among its memory operations and adds no wait of its own
// before reads of the destination, so a kernel that uses them orders every
// such read with an explicit s_waitcnt vmcnt and a barrier. M0 (the LDS
// address operand) is saved and restored around each instruction.
template <int D>
__device__ __forceinline__ void tile_dma_asm(unsigned char* lds, const void* src, uint32_t bytes, int wave,
                                             int lane) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int NI = BC<D>::TILE / 1024, RPI = 1024 / BC<D>::RB;
    static_assert(NI % 4 == 0 && kThreads == 256, "four waves share a tile's DMA instructions");
    const uint64_t a = reinterpret_cast<uint64_t>(src);
    const u32x4_t d = {(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
                       (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xFFFFu),
                       (uint32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000u};
#pragma unroll
    for (int m = 0; m < NI / 4; ++m) {
        const int n = wave * (NI / 4) + m;
        const int row = RPI * n + lane / BC<D>::CH, pos = lane % BC<D>::CH;
        const uint32_t voff = (uint32_t)(row * BC<D>::RB + 16 * (pos ^ swz<D>(row)));
        const uint32_t la = __builtin_amdgcn_readfirstlane(
            (uint32_t)(size_t)(__attribute__((address_space(3))) unsigned char*)(lds + 1024 * n));
        uint32_t saved;
        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                     "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                     : "=&s"(saved) : "s"(la), "v"(voff), "s"(d) : "memory");
    }
}

struct VirtRow {
    const uint32_t* mrow;
    const float* wrow;
    int N;
    float lnlast2;
    __device__ float bias(int j, bool with_mass) const {
        if (j >= N || ((mrow[j >> 5] >> (j & 31)) & 1u)) return -INFINITY;
        float b = wrow ? wrow[j] * kLog2e : 0.f;
        if (with_mass) b += j == N - 1 ? lnlast2 : 6.0f;   // log2 n_j
        return b;
    }
    __device__ float mass(int j) const { return j == N - 1 ? fexp2(lnlast2) : 64.f; }
};

// Bits j = 32 w0 .. 32 w0 + 63 of a query block's exact-set mask row (words
// w0 and w0 + 1; bits at j >= N are zero). The row is the same for the whole
// workgroup, so these are scalar loads and a loop over the set bits skips
// the blocks that are not exact without touching them.
__device__ __forceinline__ uint64_t mask_pair(const uint32_t* mrow, int w0, int NW) {
    uint64_t b = mrow[w0];
    if (w0 + 1 < NW) b |= (uint64_t)mrow[w0 + 1] << 32;
    return b;
}

// (H g)^T for the head-dim tiles [dt0, dt0 + D / 64): A = H rows (hi + lo), B = dout rows.
template <int D, typename BOp>
__device__ __forceinline__ void hg_tiles(f32x16_t (&hg)[D / 64], const bf16_t* hh, const bf16_t* hl, BOp bop,
                                         int dt0, int r32, int g) {
#pragma unroll
    for (int x = 0; x < D / 64; ++x) {
        f32x16_t c = zero16();
        const int d = (dt0 + x) * 32 + r32;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const int64_t o = (int64_t)d * D + 16 * ks + 8 * g;
            const bf16x8_t b = bop(ks);
            c = mfma(as_bf16x8(*reinterpret_cast<const uint4*>(hh + o)), b, c);
            c = mfma(as_bf16x8(*reinterpret_cast<const uint4*>(hl + o)), b, c);
        }
        hg[x] = c;
    }
}

// ---------------------------------------------------------------- row statistics
// Per query row: lse over the exact keys and the virtual tokens (mass n_j),
// delta = dout . o, beta = dout . (q' H) / T and c = l_tail / (T den).
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void bwd_rowstats_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ o,
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ kbh, const bf16_t* __restrict__ kbl,
    const bf16_t* __restrict__ hh, const bf16_t* __restrict__ hl, const uint32_t* __restrict__ mask,
    const float* __restrict__ wgate, f32x4_t* __restrict__ rowstat, int T, int N, int NW, float scale,
    int second_order, int first_order) {
    using C = BC<D>;
    __shared__ __attribute__((aligned(16))) unsigned char sK[C::TILE];
    __shared__ float sx[2][32][4];
    __shared__ __attribute__((aligned(16))) float sbias[64];   // a group's virtual-token biases (log2)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, g = lane >> 5;
    const int kt = wave >> 1, qt = wave & 1;
    int i;
    int64_t bh;
    xcd_tile(&i, &bh);
    const int t = i * kBlock + qt * 32 + r32;
    const int64_t base = bh * (int64_t)T * D;
    const uint32_t* mrow = mask + (bh * N + i) * (int64_t)NW;
    const float c2 = scale * kLog2e;
    const VirtRow vr{mrow, second_order ? wgate + (bh * N + i) * (int64_t)N : nullptr, N,
                     log2f((float)(T - (N - 1) * kBlock))};

    uint4 qreg[C::KS];
    rows_from_global<D>(qreg, q + base, t, T, g);
    float m = -INFINITY, l = 0.f, lt = 0.f;   // log2-domain max; sums against it
    auto merge = [&](const f32x16_t& z, bool tail) {
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, z[r]);
        if (mx == -INFINITY) return;
        const float mn = fmaxf(m, mx);
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) a += fexp2(z[r] - mn);
        const float cr = m == -INFINITY ? 0.f : fexp2(m - mn);
        l = l * cr + a;
        lt = lt * cr + (tail ? a : 0.f);
        m = mn;
    };
    for (int w0 = 0; w0 < NW; w0 += 2) {   // exact KV blocks j: the set bits of the mask row
        uint64_t bits = mask_pair(mrow, w0, NW);
        while (bits) {
            const int j = 32 * w0 + __builtin_ctzll(bits);
            bits &= bits - 1;
            const int nval = min(kBlock, T - j * kBlock);
            uint4 kr[C::LPT];
            const __amdgpu_buffer_rsrc_t rk = brsrc(k + base + (int64_t)j * kBlock * D, (uint32_t)(nval * C::RB));
#pragma unroll
            for (int m = 0; m < C::LPT; ++m)
                kr[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(16 * (tid + kThreads * m)), 0, 0));
            __syncthreads();
            tile_store<D>(sK, kr, tid);
            __syncthreads();
            f32x16_t s = zero16();
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) s = mfma(row_op<D>(sK, kt * 32 + r32, ks, g), as_bf16x8(qreg[ks]), s);
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = kt * 32 + acc_row(r, g) < nval ? s[r] * c2 : -INFINITY;
            merge(s, false);
        }
    }
    const bf16_t* kbh_h = kbh + bh * (int64_t)N * D;
    const bf16_t* kbl_h = kbl + bh * (int64_t)N * D;
    for (int G = 0; G * 64 < N; ++G) {   // virtual tokens, 64 blocks at a time (rows of kbar as A)
        __syncthreads();                  // the previous group's biases have been read
        if (tid < 64) sbias[tid] = vr.bias(G * 64 + tid, true);
        __syncthreads();
        const int jr = G * 64 + kt * 32 + r32;
        f32x16_t s = zero16();
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int64_t oo = (int64_t)jr * D + 16 * ks + 8 * g;
            const uint4 ah = jr < N ? *reinterpret_cast<const uint4*>(kbh_h + oo) : make_uint4(0, 0, 0, 0);
            const uint4 al = jr < N ? *reinterpret_cast<const uint4*>(kbl_h + oo) : make_uint4(0, 0, 0, 0);
            s = mfma(as_bf16x8(ah), as_bf16x8(qreg[ks]), s);
            s = mfma(as_bf16x8(al), as_bf16x8(qreg[ks]), s);
        }
#pragma unroll
        for (int run = 0; run < 4; ++run) {   // the biases of rows 8 run + 4 g + (0..3)
            const f32x4_t b = *reinterpret_cast<const f32x4_t*>(sbias + kt * 32 + 8 * run + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) s[4 * run + e] = fmaf(s[4 * run + e], c2, b[e]);
        }
        merge(s, true);
    }
    // lanes l and l ^ 32 hold the same query
    {   // (a state with no finite logit has m = -inf and sums 0)
        const float mo = __shfl_xor(m, 32), lo_ = __shfl_xor(l, 32), to = __shfl_xor(lt, 32);
        const float mn = fmaxf(m, mo);
        const float a = m == -INFINITY ? 0.f : fexp2(m - mn), b = mo == -INFINITY ? 0.f : fexp2(mo - mn);
        l = l * a + lo_ * b;
        lt = lt * a + to * b;
        m = mn;
    }
    // beta: this wave's head-dim tiles of (H g)^T, dotted with q
    float bp = 0.f;
    if (first_order) {
        uint4 oreg[C::KS];
        rows_from_global<D>(oreg, dout + base, t, T, g);
        f32x16_t hg[C::DT / 2];
        hg_tiles<D>(hg, hh + bh * (int64_t)D * D, hl + bh * (int64_t)D * D,
                    [&](int ks) { return as_bf16x8(oreg[ks]); }, kt * C::DT / 2, r32, g);
        if (t < T) {
#pragma unroll
            for (int x = 0; x < C::DT / 2; ++x)
#pragma unroll
                for (int run = 0; run < 4; ++run) {
                    const int d0 = (kt * C::DT / 2 + x) * 32 + 8 * run + 4 * g;
                    const uint2 qq = *reinterpret_cast<const uint2*>(q + base + (int64_t)t * D + d0);
                    bp += bf16_lo(qq.x) * hg[x][4 * run] + bf16_hi(qq.x) * hg[x][4 * run + 1] +
                          bf16_lo(qq.y) * hg[x][4 * run + 2] + bf16_hi(qq.y) * hg[x][4 * run + 3];
                }
        }
        bp += __shfl_xor(bp, 32);
    }
    if (kt == 1 && g == 0) {
        sx[qt][r32][0] = m;
        sx[qt][r32][1] = l;
        sx[qt][r32][2] = lt;
        sx[qt][r32][3] = bp;
    }
    __syncthreads();
    if (kt == 0 && t < T) {
        // delta = dout . o over this lane's half of the head dims
        float dl = 0.f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
            const int d0 = (D / 2) * g + 8 * c;
            const uint4 a = *reinterpret_cast<const uint4*>(dout + base + (int64_t)t * D + d0);
            const uint4 b = *reinterpret_cast<const uint4*>(o + base + (int64_t)t * D + d0);
            dl += bf16_lo(a.x) * bf16_lo(b.x) + bf16_hi(a.x) * bf16_hi(b.x) + bf16_lo(a.y) * bf16_lo(b.y) +
                  bf16_hi(a.y) * bf16_hi(b.y) + bf16_lo(a.z) * bf16_lo(b.z) + bf16_hi(a.z) * bf16_hi(b.z) +
                  bf16_lo(a.w) * bf16_lo(b.w) + bf16_hi(a.w) * bf16_hi(b.w);
        }
        dl += __shfl_xor(dl, 32);
        if (g == 0) {
            const float mo = sx[qt][r32][0], lo_ = sx[qt][r32][1], to = sx[qt][r32][2];
            const float mn = fmaxf(m, mo);   // finite: the query's own block is exact
            const float a = m == -INFINITY ? 0.f : fexp2(m - mn), b = mo == -INFINITY ? 0.f : fexp2(mo - mn);
            const float ls = l * a + lo_ * b, ts = lt * a + to * b;
            const float beta = first_order ? scale * (bp + sx[qt][r32][3]) / (float)T : 0.f;
            const float cf = first_order ? (ts / ls) / (float)T : 0.f;
            f32x4_t rs = {(mn + log2f(ls)) * kLn2, dl, beta, cf};
            rowstat[bh * (int64_t)T + t] = rs;
        }
    }
}

// Row statistics when the forward wrote each row's lse and c (pisa_attn_fwd's
// row_stats): the exact and virtual pairs are not re-scored; only delta =
// dout . o and beta = s dout . (q H) / T are formed, as above (beta by the
// same hi + lo products of H with dout, summed over the two key halves). A
// workgroup takes kRsBlocks query blocks, so each wave loads its H operands
// (its half of the head dims, hi and lo) once for all of them.
constexpr int kRsBlocks = 8;
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rowstats_fwd_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout,
    const bf16_t* __restrict__ hh, const bf16_t* __restrict__ hl, const float* __restrict__ fwd_rstat,
    f32x4_t* __restrict__ rowstat, int T, int N, float scale, int first_order) {
    using C = BC<D>;
    constexpr int HX = C::DT / 2;
    // The Q, O and dout tiles of a query block, coalesced by buffer->LDS DMA
    // in the staged layout, two blocks deep: those of block i + 1 arrive while
    // block i is computed. The DMAs are inline asm (tile_dma_asm); every read
    // of a stage follows the explicit wait and barrier at the block's start.
    __shared__ __attribute__((aligned(16))) unsigned char st0[3 * C::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char st1[3 * C::TILE];
    __shared__ float sbp[2][32];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, g = lane >> 5;
    const int kt = wave >> 1, qt = wave & 1;
    const int64_t bh = blockIdx.y;
    const int64_t base = bh * (int64_t)T * D;
    const int i0 = blockIdx.x * kRsBlocks, i1 = min(N, i0 + kRsBlocks);
    bf16x8_t ha[HX][C::KS], la[HX][C::KS];   // A = H rows (hi, lo) of this wave's head-dim tiles
    if (first_order) {
#pragma unroll
        for (int x = 0; x < HX; ++x)
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int64_t a = bh * (int64_t)D * D + (int64_t)((kt * HX + x) * 32 + r32) * D + 16 * ks + 8 * g;
                ha[x][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(hh + a));
                la[x][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(hl + a));
            }
    }
    // the H operands have landed (an s_waitcnt vmcnt(0) the compiler sees, so
    // that it issues no waits of its own for them inside the loop, where they
    // would also wait for the tile DMAs in flight)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    auto dma_block = [&](int i, unsigned char* stg) {
        const int rows = min(kBlock, T - i * kBlock);
        const uint32_t bytes = (uint32_t)(rows * C::RB);
        const int64_t off = base + (int64_t)i * kBlock * D;
        tile_dma_asm<D>(stg, q + off, bytes, wave, lane);
        tile_dma_asm<D>(stg + C::TILE, o + off, bytes, wave, lane);
        tile_dma_asm<D>(stg + 2 * C::TILE, dout + off, bytes, wave, lane);
    };
    // 8 bytes (4 bf16: head dims d0 .. d0 + 3, d0 % 4 = 0) of row rr of a staged tile
    auto row8 = [&](const unsigned char* tile, int rr, int d0) {
        return *reinterpret_cast<const uint2*>(tile + rr * C::RB + 16 * ((d0 >> 3) ^ swz<D>(rr)) + 2 * (d0 & 7));
    };
    if (i0 < i1) dma_block(i0, st0);
    auto body = [&](auto par, int i) {
        constexpr int PAR = decltype(par)::value;
        const unsigned char* sQ = PAR == 0 ? st0 : st1;
        const unsigned char* sO = sQ + C::TILE;
        const unsigned char* sG = sQ + 2 * C::TILE;
        const int rr = qt * 32 + r32;
        const int t = i * kBlock + rr;
        float2 fr = {0.f, 0.f};
        if (kt == 0 && g == 0 && t < T) fr = *reinterpret_cast<const float2*>(fwd_rstat + 2 * (bh * (int64_t)T + t));
        // this wave's DMAs of block i (and every earlier load) have landed;
        // after the barrier every wave's have, every wave is done with the
        // other stage and with the previous block's partial sums
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : "+v"(fr.x), "+v"(fr.y) : : "memory");
        if (i + 1 < i1) dma_block(i + 1, PAR == 0 ? st1 : st0);
        float bp = 0.f;
        if (first_order) {
            f32x16_t hg[HX];
#pragma unroll
            for (int x = 0; x < HX; ++x) {
                f32x16_t c = zero16();
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const bf16x8_t b = row_op<D>(sG, rr, ks, g);
                    c = mfma(ha[x][ks], b, c);
                    c = mfma(la[x][ks], b, c);
                }
                hg[x] = c;
            }
            if (t < T) {
#pragma unroll
                for (int x = 0; x < HX; ++x)
#pragma unroll
                    for (int run = 0; run < 4; ++run) {
                        const int d0 = (kt * HX + x) * 32 + 8 * run + 4 * g;
                        const uint2 qq = row8(sQ, rr, d0);
                        bp += bf16_lo(qq.x) * hg[x][4 * run] + bf16_hi(qq.x) * hg[x][4 * run + 1] +
                              bf16_lo(qq.y) * hg[x][4 * run + 2] + bf16_hi(qq.y) * hg[x][4 * run + 3];
                    }
            }
            bp += __shfl_xor(bp, 32);
        }
        if (kt == 1 && g == 0) sbp[qt][r32] = bp;
        __syncthreads();
        if (kt == 0 && t < T) {
            float dl = 0.f;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const int d0 = (D / 2) * g + 8 * c;
                const uint2 a0 = row8(sG, rr, d0), a1 = row8(sG, rr, d0 + 4);
                const uint2 b0 = row8(sO, rr, d0), b1 = row8(sO, rr, d0 + 4);
                const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y), b = make_uint4(b0.x, b0.y, b1.x, b1.y);
                dl += bf16_lo(a.x) * bf16_lo(b.x) + bf16_hi(a.x) * bf16_hi(b.x) + bf16_lo(a.y) * bf16_lo(b.y) +
                      bf16_hi(a.y) * bf16_hi(b.y) + bf16_lo(a.z) * bf16_lo(b.z) + bf16_hi(a.z) * bf16_hi(b.z) +
                      bf16_lo(a.w) * bf16_lo(b.w) + bf16_hi(a.w) * bf16_hi(b.w);
            }
            dl += __shfl_xor(dl, 32);
            if (g == 0) {
                const float beta = first_order ? scale * (bp + sbp[qt][r32]) / (float)T : 0.f;
                f32x4_t rs = {fr.x, dl, beta, first_order ? fr.y : 0.f};
                rowstat[bh * (int64_t)T + t] = rs;
            }
        }
    };
    for (int i = i0; i < i1; i += 2) {
        body(std::integral_constant<int, 0>(), i);
        if (i + 1 < i1) body(std::integral_constant<int, 1>(), i + 1);
    }
}

// ---------------------------------------------------------------- dH
// dH = sum_t (c_t s q_t)^T dout_t over one range of rows (a partial sum; the
// ranges are added in a fixed order afterwards), on the matrix cores: the Q
// and dO tiles are staged in LDS and read transposed, which gives both
// operands the same rows in the same k-slots; A = Q^T (exact in bf16), B =
// dO^T with each row scaled by c_t s, split into bf16 hi + lo (two products).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_dh_mfma_kernel(const bf16_t* __restrict__ q,
                                                               const bf16_t* __restrict__ dout,
                                                               const f32x4_t* __restrict__ rowstat,
                                                               float* __restrict__ part, int T, int rows_per,
                                                               float scale) {
    using C = BC<D>;
    constexpr int TPW = C::DT * C::DT / 4;   // 32 x 32 output tiles per wave
    __shared__ __attribute__((aligned(16))) unsigned char sq[C::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char so[C::TILE];
    __shared__ float sc[64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, g = lane >> 5;
    const int64_t bh = blockIdx.y;
    const int64_t base = bh * (int64_t)T * D;
    const int t0 = blockIdx.x * rows_per, t1 = min(T, t0 + rows_per);
    const TrAddr ta(lane, C::RB, C::SWM);
    f32x16_t acc[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) acc[x] = zero16();
    for (int ts = t0; ts < t1; ts += kBlock) {
        const int nh = min(kBlock, t1 - ts);
        uint4 qr[C::LPT], orr[C::LPT];
        tile_load<D>(qr, q + base + (int64_t)ts * D, nh, tid);
        tile_load<D>(orr, dout + base + (int64_t)ts * D, nh, tid);
        const float cst = tid < nh ? rowstat[bh * (int64_t)T + ts + tid][3] * scale : 0.f;
        __syncthreads();   // the previous tiles have been read
        tile_store<D>(sq, qr, tid);
        tile_store<D>(so, orr, tid);
        if (tid < kBlock) sc[tid] = cst;
        __syncthreads();
#pragma unroll
        for (int r0 = 0; r0 < kBlock; r0 += 16) {
            float cs[8];   // k-slots 0..3: rows r0 + 4g + e; 4..7: rows r0 + 8 + 4g + e
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                cs[e] = sc[r0 + 4 * g + e];
                cs[4 + e] = sc[r0 + 8 + 4 * g + e];
            }
#pragma unroll
            for (int x = 0; x < TPW; ++x) {
                const int u = wave * TPW + x, da = u / C::DT, db = u % C::DT;
                const bf16x8_t a = tr_op<D>(sq, ta, da, r0);
                const uint4 bw = __builtin_bit_cast(uint4, tr_op<D>(so, ta, db, r0));
                const uint32_t w[4] = {bw.x, bw.y, bw.z, bw.w};
                f32x16_t bs;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bs[2 * e] = bf16_lo(w[e]) * cs[2 * e];
                    bs[2 * e + 1] = bf16_hi(w[e]) * cs[2 * e + 1];
                }
                bf16x8_t bhi, blo;
                split_op(bs, 0, bhi, blo);
                acc[x] = mfma(a, bhi, acc[x]);
                acc[x] = mfma(a, blo, acc[x]);
            }
        }
    }
    float* out = part + (bh * gridDim.x + blockIdx.x) * (int64_t)D * D;
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int u = wave * TPW + x, da = u / C::DT, db = u % C::DT;
#pragma unroll
        for (int i = 0; i < 16; ++i) out[(da * 32 + acc_row(i, g)) * D + db * 32 + r32] = acc[x][i];
    }
}

// ---------------------------------------------------------------- dq
// dq' = K^T dS^T (exact keys) + kbar^T dlam^T (virtual tokens, kbar hi + lo)
// + c H g, then dq = s dq' + 2 s^2 q dq2bar_i / n_i (second order).
// Q and dO of the query block sit in LDS (B operands), so that a wave fits
// in 256 registers and two waves share a SIMD.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ kbh, const bf16_t* __restrict__ kbl,
    const bf16_t* __restrict__ vhh, const bf16_t* __restrict__ vhl, const bf16_t* __restrict__ hh,
    const bf16_t* __restrict__ hl, const uint32_t* __restrict__ mask, const float* __restrict__ wgate,
    const f32x4_t* __restrict__ rowstat, const float* __restrict__ dq2, bf16_t* __restrict__ dq, int T, int N,
    int NW, float scale, int second_order, int first_order) {
    using C = BC<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::TILE];   // K, V (or kbar hi, lo) tiles; exchange
    __shared__ __attribute__((aligned(16))) float sbias[64], smass[64];      // a virtual group's biases, n_j
    __shared__ __attribute__((aligned(16))) unsigned char sqo[2 * C::TILE];   // Q, dO of the query block
    unsigned char* sK = smem;
    unsigned char* sV = smem + C::TILE;
    unsigned char* sQt = sqo;
    unsigned char* sOt = sqo + C::TILE;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, g = lane >> 5;
    const int kt = wave >> 1, qt = wave & 1;
    int i;
    int64_t bh;
    xcd_tile(&i, &bh);
    const int t = i * kBlock + qt * 32 + r32;
    const int64_t base = bh * (int64_t)T * D;
    const uint32_t* mrow = mask + (bh * N + i) * (int64_t)NW;
    const float c2 = scale * kLog2e;
    const TrAddr ta(lane, C::RB, C::SWM);
    const VirtRow vr{mrow, second_order ? wgate + (bh * N + i) * (int64_t)N : nullptr, N,
                     log2f((float)(T - (N - 1) * kBlock))};

    {
        const int rows = min(kBlock, T - i * kBlock);
        uint4 a_[C::LPT], b_[C::LPT];
        tile_load<D>(a_, q + base + (int64_t)i * kBlock * D, rows, tid);
        tile_load<D>(b_, dout + base + (int64_t)i * kBlock * D, rows, tid);
        tile_store<D>(sQt, a_, tid);
        tile_store<D>(sOt, b_, tid);
    }
    // B operands: this lane's query row, head dims 16 ks + 8 g ..
    auto qop = [&](int ks) { return row_op<D>(sQt, qt * 32 + r32, ks, g); };
    auto oop = [&](int ks) { return row_op<D>(sOt, qt * 32 + r32, ks, g); };
    float lse2 = INFINITY, delta = 0.f, beta = 0.f, cf = 0.f;
    if (t < T) {
        const f32x4_t rs = rowstat[bh * (int64_t)T + t];
        lse2 = rs[0] * kLog2e;
        delta = rs[1];
        beta = rs[2];
        cf = rs[3];
    }
    f32x16_t acc[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) acc[dt] = zero16();

    // exact KV blocks j: the set bits of the mask row, in ascending order; the
    // K and V tiles of the next one load into registers while this one's
    // products run
    int w0 = 0;
    uint64_t bits = mask_pair(mrow, 0, NW);
    auto next_exact = [&]() {   // the next exact block, or -1
        while (bits == 0) {
            w0 += 2;
            if (w0 >= NW) return -1;
            bits = mask_pair(mrow, w0, NW);
        }
        const int jn = 32 * w0 + __builtin_ctzll(bits);
        bits &= bits - 1;
        return jn;
    };
    uint4 kr[C::LPT], vr_[C::LPT];
    auto load_kv = [&](int jl) {
        const int nl = min(kBlock, T - jl * kBlock);
        const __amdgpu_buffer_rsrc_t rk = brsrc(k + base + (int64_t)jl * kBlock * D, (uint32_t)(nl * C::RB));
        const __amdgpu_buffer_rsrc_t rv = brsrc(v + base + (int64_t)jl * kBlock * D, (uint32_t)(nl * C::RB));
#pragma unroll
        for (int m = 0; m < C::LPT; ++m) {
            const uint32_t o = (uint32_t)(16 * (tid + kThreads * m));
            kr[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)o, 0, 0));
            vr_[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)o, 0, 0));
        }
    };
    int j = next_exact();
    if (j >= 0) load_kv(j);
    while (j >= 0) {
        {
            const int nval = min(kBlock, T - j * kBlock);
            __syncthreads();
            tile_store<D>(sK, kr, tid);
            tile_store<D>(sV, vr_, tid);
            __syncthreads();
            const int jn = next_exact();
            if (jn >= 0) load_kv(jn);
            f32x16_t s = zero16(), dp = zero16();
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                s = mfma(row_op<D>(sK, kt * 32 + r32, ks, g), qop(ks), s);
                dp = mfma(row_op<D>(sV, kt * 32 + r32, ks, g), oop(ks), dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = kt * 32 + acc_row(r, g) < nval ? fexp2(fmaf(s[r], c2, -lse2)) : 0.f;
                s[r] = p * (dp[r] - delta);   // dS^T
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                bf16x8_t hi, lo;
                split_op(s, h, hi, lo);
                const int r0 = kt * 32 + 16 * h;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const bf16x8_t a = tr_op<D>(sK, ta, dt, r0);   // K^T: head dims x keys
                    acc[dt] = mfma(a, hi, acc[dt]);
                    acc[dt] = mfma(a, lo, acc[dt]);
                }
            }
            j = jn;
        }
    }
    // virtual tokens, 64 blocks at a time: kbar hi / lo tiles in LDS
    const bf16_t* kbh_h = kbh + bh * (int64_t)N * D;
    const bf16_t* kbl_h = kbl + bh * (int64_t)N * D;
    const bf16_t* vhh_h = vhh + bh * (int64_t)N * D;
    const bf16_t* vhl_h = vhl + bh * (int64_t)N * D;
    for (int G = 0; G * 64 < N; ++G) {
        const int nb = min(64, N - G * 64);
        uint4 kr[C::LPT], kl[C::LPT];
        tile_load<D>(kr, kbh_h + (int64_t)G * 64 * D, nb, tid);
        tile_load<D>(kl, kbl_h + (int64_t)G * 64 * D, nb, tid);
        __syncthreads();
        tile_store<D>(sK, kr, tid);
        tile_store<D>(sV, kl, tid);
        if (tid < 64) {
            const int jj = G * 64 + tid;
            sbias[tid] = vr.bias(jj, false);
            smass[tid] = jj < N ? vr.mass(jj) : 0.f;
        }
        __syncthreads();
        const int jr = G * 64 + kt * 32 + r32;
        f32x16_t s = zero16(), gv = zero16();
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const bf16x8_t ah = row_op<D>(sK, kt * 32 + r32, ks, g), al = row_op<D>(sV, kt * 32 + r32, ks, g);
            const bf16x8_t bq = qop(ks);
            s = mfma(ah, bq, s);
            s = mfma(al, bq, s);
            const int64_t oo = (int64_t)jr * D + 16 * ks + 8 * g;
            const uint4 vh = jr < N ? *reinterpret_cast<const uint4*>(vhh_h + oo) : make_uint4(0, 0, 0, 0);
            const uint4 vl = jr < N ? *reinterpret_cast<const uint4*>(vhl_h + oo) : make_uint4(0, 0, 0, 0);
            const bf16x8_t bo = oop(ks);
            gv = mfma(as_bf16x8(vh), bo, gv);
            gv = mfma(as_bf16x8(vl), bo, gv);
        }
#pragma unroll
        for (int run = 0; run < 4; ++run) {   // blocks 8 run + 4 g + (0..3) of the key half kt
            const f32x4_t b = *reinterpret_cast<const f32x4_t*>(sbias + kt * 32 + 8 * run + 4 * g);
            const f32x4_t nm = *reinterpret_cast<const f32x4_t*>(smass + kt * 32 + 8 * run + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * run + e;
                const float a = b[e] == -INFINITY ? 0.f : fexp2(fmaf(s[r], c2, b[e] - lse2));
                s[r] = a * (gv[r] + nm[e] * (beta - delta));   // dlam^T
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8_t dh, dlo;
            split_op(s, h, dh, dlo);
            const int r0 = kt * 32 + 16 * h;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const bf16x8_t ah = tr_op<D>(sK, ta, dt, r0), al = tr_op<D>(sV, ta, dt, r0);   // kbar^T
                acc[dt] = mfma(ah, dh, acc[dt]);
                acc[dt] = mfma(ah, dlo, acc[dt]);
                acc[dt] = mfma(al, dh, acc[dt]);
            }
        }
    }
    // c H g on this wave's head-dim tiles
    if (first_order) {
        f32x16_t hg[C::DT / 2];
        hg_tiles<D>(hg, hh + bh * (int64_t)D * D, hl + bh * (int64_t)D * D, oop, kt * C::DT / 2, r32, g);
        // tile dt belongs to wave kt = dt / (DT / 2): compile-time indices, a runtime select
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
            if (dt / (C::DT / 2) == kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] = fmaf(cf, hg[dt % (C::DT / 2)][r], acc[dt][r]);
    }
    // the two key halves of each query tile: wave (1, qt) hands its partial to wave (0, qt)
    __syncthreads();
    float* xs = reinterpret_cast<float*>(smem);   // [qt][dt][16][64]: 2 * DT * 4 KB = 2 tiles
    if (kt == 1) {
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) xs[((qt * C::DT + dt) * 16 + r) * 64 + lane] = acc[dt][r];
    }
    __syncthreads();
    if (kt == 0 && t < T) {
        const int rows = min(kBlock, T - i * kBlock);
        const float c2o = second_order ? 2.f * scale * scale / (float)rows : 0.f;
        const float* q2 = second_order ? dq2 + (bh * N + i) * (int64_t)D : nullptr;
        bf16_t* out = dq + base + (int64_t)t * D;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int run = 0; run < 4; ++run) {
                const int d0 = dt * 32 + 8 * run + 4 * g;
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * run + e;
                    x[e] = scale * (acc[dt][r] + xs[((qt * C::DT + dt) * 16 + r) * 64 + lane]);
                }
                if (second_order) {
                    const uint2 qq = *reinterpret_cast<const uint2*>(q + base + (int64_t)t * D + d0);
                    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(q2 + d0);
                    x[0] = fmaf(c2o * bf16_lo(qq.x), w[0], x[0]);
                    x[1] = fmaf(c2o * bf16_hi(qq.x), w[1], x[1]);
                    x[2] = fmaf(c2o * bf16_lo(qq.y), w[2], x[2]);
                    x[3] = fmaf(c2o * bf16_hi(qq.y), w[3], x[3]);
                }
                const uint32_t w0 = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
                const uint32_t w1 = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
                *reinterpret_cast<uint2*>(out + d0) = make_uint2(w0, w1);
            }
    }
}

// dq2bar_i = 1/2 sum_j dW_ij sig2_j (dW is 0 for gated and exact pairs).
__global__ __launch_bounds__(128) void bwd_dq2_kernel(const float* __restrict__ dw, const double* __restrict__ ksig2,
                                                      float* __restrict__ dq2, int N, int D) {
    const int i = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const float* row = dw + (bh * N + i) * (int64_t)N;
    for (int d = threadIdx.x; d < D; d += 128) {
        float acc = 0.f;
        for (int j = 0; j < N; ++j) acc = fmaf(row[j], (float)ksig2[(bh * N + j) * (int64_t)D + d], acc);
        dq2[(bh * N + i) * (int64_t)D + d] = 0.5f * acc;
    }
}

// ---------------------------------------------------------------- dk, dv exact
// K and V of the block sit in LDS (read as B operands each step) rather than
// in registers, so that a wave fits in 256 registers and two waves share a
// SIMD: one wave's LDS waits overlap the other's products.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_exact_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const uint32_t* __restrict__ mask, const f32x4_t* __restrict__ rowstat,
    const double* __restrict__ kbar, const float* __restrict__ vsum, const float* __restrict__ dH,
    const float* __restrict__ dHT, const float* __restrict__ dkb_part, const float* __restrict__ dvh_part,
    const float* __restrict__ dsg, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int T, int N, int NW,
    float scale, int nsplit, int second_order, int first_order) {
    using C = BC<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * C::TILE];   // Q, dO tiles; then the exchange
    __shared__ __attribute__((aligned(16))) unsigned char skv[2 * C::TILE];    // K, V of the block
    __shared__ float slse[64], sdel[64];
    __shared__ float sblk[5][D];   // the block's kbar, dkbar, dV-hat, dsig2, dH V-hat
    __shared__ uint32_t scol[kThreads / 32];   // selection bits of kThreads query blocks
    unsigned char* sQ = smem;
    unsigned char* sO = smem + C::TILE;
    unsigned char* sKt = skv;
    unsigned char* sVt = skv + C::TILE;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, g = lane >> 5;
    const int kt = wave >> 1, qt = wave & 1;
    int j;
    int64_t bh;
    xcd_tile(&j, &bh);
    const int key = j * kBlock + kt * 32 + r32;
    const int64_t base = bh * (int64_t)T * D;
    const float c2 = scale * kLog2e;
    const TrAddr ta(lane, C::RB, C::SWM);

    {
        const int nval = min(kBlock, T - j * kBlock);
        uint4 kr[C::LPT], vr_[C::LPT];
        tile_load<D>(kr, k + base + (int64_t)j * kBlock * D, nval, tid);
        tile_load<D>(vr_, v + base + (int64_t)j * kBlock * D, nval, tid);
        tile_store<D>(sKt, kr, tid);
        tile_store<D>(sVt, vr_, tid);
    }
    f32x16_t dva[C::DT], dka[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) dva[dt] = dka[dt] = zero16();

    // query blocks whose exact set holds j, kThreads at a time: one mask word per
    // thread, the selections gathered by ballot; the set bits are then walked in order
    for (int i0 = 0; i0 < N; i0 += kThreads) {
        const bool sel = i0 + tid < N &&
                         ((mask[(bh * N + i0 + tid) * (int64_t)NW + (j >> 5)] >> (j & 31)) & 1u);
        const uint64_t bal = __ballot(sel);
        __syncthreads();   // the previous chunk's words have been read
        if (lane == 0) {
            scol[2 * wave] = (uint32_t)bal;
            scol[2 * wave + 1] = (uint32_t)(bal >> 32);
        }
        __syncthreads();
        for (int w0 = 0; w0 < kThreads / 32; w0 += 2) {
            // (readfirstlane returns int: through uint32_t, so the low word is not sign-extended)
            uint64_t bits = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(scol[w0]) |
                            ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(scol[w0 + 1]) << 32);
            while (bits) {
                const int i = i0 + 32 * w0 + __builtin_ctzll(bits);
                bits &= bits - 1;
                const int rows = min(kBlock, T - i * kBlock);
                uint4 qr[C::LPT], orr[C::LPT];
                const __amdgpu_buffer_rsrc_t rq = brsrc(q + base + (int64_t)i * kBlock * D, (uint32_t)(rows * C::RB));
                const __amdgpu_buffer_rsrc_t ro = brsrc(dout + base + (int64_t)i * kBlock * D, (uint32_t)(rows * C::RB));
#pragma unroll
                for (int m = 0; m < C::LPT; ++m) {
                    const uint32_t o = (uint32_t)(16 * (tid + kThreads * m));
                    qr[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)o, 0, 0));
                    orr[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ro, (int)o, 0, 0));
                }
                const f32x4_t rs = rowstat[bh * (int64_t)T + (int64_t)i * kBlock + min(tid & 63, rows - 1)];
                const bool in = (tid & 63) < rows;
                const float ls = in ? rs[0] * kLog2e : INFINITY;
                const float dl = in ? rs[1] : 0.f;
                __syncthreads();
                tile_store<D>(sQ, qr, tid);
                tile_store<D>(sO, orr, tid);
                if (tid < 64) {
                    slse[tid] = ls;
                    sdel[tid] = dl;
                }
                __syncthreads();
                f32x16_t s = zero16(), dp = zero16();
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    s = mfma(row_op<D>(sQ, qt * 32 + r32, ks, g), row_op<D>(sKt, kt * 32 + r32, ks, g), s);   // S
                    dp = mfma(row_op<D>(sO, qt * 32 + r32, ks, g), row_op<D>(sVt, kt * 32 + r32, ks, g), dp); // dP
                }
                f32x16_t p;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int qq = qt * 32 + acc_row(r, g);
                    p[r] = fexp2(fmaf(s[r], c2, -slse[qq]));       // rows past T: lse = +inf, P = 0
                    s[r] = p[r] * (dp[r] - sdel[qq]);              // dS
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    bf16x8_t phi, plo, hi, lo;
                    split_op(p, h, phi, plo);
                    split_op(s, h, hi, lo);
                    const int r0 = qt * 32 + 16 * h;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt) {
                        const bf16x8_t ao = tr_op<D>(sO, ta, dt, r0);            // dO^T P
                        dva[dt] = mfma(ao, phi, dva[dt]);
                        dva[dt] = mfma(ao, plo, dva[dt]);
                        const bf16x8_t aq = tr_op<D>(sQ, ta, dt, r0);            // Q^T dS
                        dka[dt] = mfma(aq, hi, dka[dt]);
                        dka[dt] = mfma(aq, lo, dka[dt]);
                    }
                }
            }
        }
    }
    // ---- epilogue. The two query halves of a key tile swap partials, so that
    // wave (kt, qt) holds the sums of head-dim tiles [qt HT, qt HT + HT); then
    // it adds the chain terms of the block and stores dk, dv:
    //   dk = s sum_t dS q + dH v + (dkbar_j - dH V-hat_j) / n_j + 2 dsig2_j (k - kbar_j) / n_j,
    //   dv = sum_t P dout + dH^T (k - kbar_j) + dV-hat_j.
    constexpr int HT = C::DT / 2;
    f32x16_t ov[HT], ok_[HT];
    float* xs = reinterpret_cast<float*>(smem);   // [kt][qt][x][16][64]: 4 * HT * 4 KB = 2 tiles
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        f32x16_t* a = pass == 0 ? dva : dka;
        f32x16_t* own = pass == 0 ? ov : ok_;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < HT; ++x) {
            const f32x16_t lo_ = a[x], hi_ = a[HT + x];
            const f32x16_t send = qt == 0 ? hi_ : lo_;
            own[x] = qt == 0 ? lo_ : hi_;
#pragma unroll
            for (int r = 0; r < 16; ++r) xs[(((kt * 2 + qt) * HT + x) * 16 + r) * 64 + lane] = send[r];
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < HT; ++x)
#pragma unroll
            for (int r = 0; r < 16; ++r) own[x][r] += xs[(((kt * 2 + (1 - qt)) * HT + x) * 16 + r) * 64 + lane];
    }
    const int64_t jb = (bh * N + j) * (int64_t)D;
    const int64_t pstride = (int64_t)gridDim.y * N * D;
    for (int d = tid; d < D; d += kThreads) {
        float sk_ = 0.f, sv_ = 0.f;
        for (int sp = 0; sp < nsplit; ++sp) {
            sk_ += dkb_part[sp * pstride + jb + d];
            sv_ += dvh_part[sp * pstride + jb + d];
        }
        float xh = 0.f;
        if (first_order) {
            const float* hr = dH + bh * (int64_t)D * D + (int64_t)d * D;
            for (int e = 0; e < D; ++e) xh = fmaf(hr[e], vsum[jb + e], xh);
        }
        sblk[0][d] = (float)kbar[jb + d];
        sblk[1][d] = sk_;
        sblk[2][d] = sv_;
        sblk[3][d] = second_order ? dsg[jb + d] : 0.f;
        sblk[4][d] = xh;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < HT; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) ok_[x][r] *= scale;
    if (first_order) {
        const float* dHh = dH + bh * (int64_t)D * D;
        const float* dHTh = dHT + bh * (int64_t)D * D;
        auto split8 = [&](const float* src, bf16x8_t& hi, bf16x8_t& lo) {
            const f32x4_t u0 = *reinterpret_cast<const f32x4_t*>(src), u1 = *reinterpret_cast<const f32x4_t*>(src + 4);
            f32x16_t t = zero16();
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = u0[e];
                t[4 + e] = u1[e];
            }
            split_op(t, 0, hi, lo);
        };
#pragma unroll
        for (int x = 0; x < HT; ++x) {
            const int row = (qt * HT + x) * 32 + r32;   // head dim of this lane's A row
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const int c0 = 16 * ks + 8 * g;
                bf16x8_t ah, al;
                // dK^T += dH V^T: A = dH rows, B = V rows of the block
                split8(dHh + (int64_t)row * D + c0, ah, al);
                const bf16x8_t bv = row_op<D>(sVt, kt * 32 + r32, ks, g);
                ok_[x] = mfma(ah, bv, ok_[x]);
                ok_[x] = mfma(al, bv, ok_[x]);
                // dV^T += dH^T (K - kbar)^T: A = dH^T rows, B = (k - kbar) of the block, hi + lo
                split8(dHTh + (int64_t)row * D + c0, ah, al);
                const uint4 kb = *reinterpret_cast<const uint4*>(sKt + (kt * 32 + r32) * C::RB +
                                                                   16 * ((2 * ks + g) ^ swz<D>(kt * 32 + r32)));
                f32x16_t kc = zero16();
                const uint32_t kw[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kc[2 * e] = bf16_lo(kw[e]) - sblk[0][c0 + 2 * e];
                    kc[2 * e + 1] = bf16_hi(kw[e]) - sblk[0][c0 + 2 * e + 1];
                }
                bf16x8_t kh, kl;
                split_op(kc, 0, kh, kl);
                ov[x] = mfma(ah, kh, ov[x]);
                ov[x] = mfma(ah, kl, ov[x]);
                ov[x] = mfma(al, kh, ov[x]);
            }
        }
    }
    if (key < T) {
        const int nj = min(kBlock, T - j * kBlock);
        const float inv_n = 1.f / (float)nj;
        const unsigned char* krow = sKt + (kt * 32 + r32) * C::RB;
        const int sw = swz<D>(kt * 32 + r32);
#pragma unroll
        for (int x = 0; x < HT; ++x)
#pragma unroll
            for (int run = 0; run < 4; ++run) {
                const int d0 = (qt * HT + x) * 32 + 8 * run + 4 * g;
                // k of this key at dims d0 .. d0 + 3 (one 8-byte piece of its chunk)
                const uint2 kk = *reinterpret_cast<const uint2*>(krow + 16 * ((d0 >> 3) ^ sw) + 2 * (d0 & 7));
                const float kv[4] = {bf16_lo(kk.x), bf16_hi(kk.x), bf16_lo(kk.y), bf16_hi(kk.y)};
                float gk[4], gv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = d0 + e, r = 4 * run + e;
                    gk[e] = ok_[x][r] + (sblk[1][d] - sblk[4][d]) * inv_n;
                    if (second_order) gk[e] = fmaf(2.f * sblk[3][d] * inv_n, kv[e] - sblk[0][d], gk[e]);
                    gv[e] = ov[x][r] + sblk[2][d];
                }
                const int64_t o = base + (int64_t)key * D + d0;
                *reinterpret_cast<uint2*>(dk + o) =
                    make_uint2((uint32_t)f32_to_bf16(gk[0]) | ((uint32_t)f32_to_bf16(gk[1]) << 16),
                               (uint32_t)f32_to_bf16(gk[2]) | ((uint32_t)f32_to_bf16(gk[3]) << 16));
                *reinterpret_cast<uint2*>(dv + o) =
                    make_uint2((uint32_t)f32_to_bf16(gv[0]) | ((uint32_t)f32_to_bf16(gv[1]) << 16),
                               (uint32_t)f32_to_bf16(gv[2]) | ((uint32_t)f32_to_bf16(gv[3]) << 16));
            }
    }
}

// ---------------------------------------------------------------- virtual tokens
// One workgroup per (bh, group of 64 KV blocks, query split): the blocks'
// virtual tokens (key kbar_j, value V-hat_j, both fp32 split into bf16 hi +
// lo) against the query blocks of the split for which they are virtual.
//   Lam = Q kbar^T, GV = dO V-hat^T (queries on registers, blocks on lanes),
//   A = exp(s Lam + w_ij - lse), dlam = A (GV + n_j (beta - delta)),
//   dkbar^T += Q^T dlam (times s), dV-hat^T += dO^T A,
//   dW_ij = sum over the query block's rows of dlam (0 for gated pairs).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_virt_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout, const double* __restrict__ kbar,
    const float* __restrict__ vsum, const uint32_t* __restrict__ mask, const f32x4_t* __restrict__ rowstat,
    const float* __restrict__ wgate, float* __restrict__ dkb_part, float* __restrict__ dvh_part,
    float* __restrict__ dw, int T, int N, int NW, float scale, int second_order, int i_per_split) {
    using C = BC<D>;
    // The Q and dO tiles and the row statistics of two consecutive query
    // blocks live in separate arrays: those of block i + 1 arrive by
    // buffer->LDS DMA while block i is computed (separate arrays, so that the
    // compiler can tell the DMA into one from the reads of the other). The
    // partial exchange at the end reuses tqo0.
    __shared__ __attribute__((aligned(16))) unsigned char tqo0[2 * C::TILE];
    __shared__ __attribute__((aligned(16))) unsigned char tqo1[2 * C::TILE];
    __shared__ __attribute__((aligned(16))) f32x4_t trs0[64];
    __shared__ __attribute__((aligned(16))) f32x4_t trs1[64];
    __shared__ float sdw[2][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, g = lane >> 5;
    const int kt = wave >> 1, qt = wave & 1;
    int gx, zs;   // group, query-range split
    int64_t bh;
    xcd_tile(&gx, &bh, &zs);
    const int g0 = gx * 64;   // the group's first block
    const int j = g0 + kt * 32 + r32;
    const bool jvalid = j < N;
    const int jc = jvalid ? j : N - 1;
    const float nj = (float)min(kBlock, T - jc * kBlock);
    const int64_t base = bh * (int64_t)T * D;
    const float c2 = scale * kLog2e;
    const TrAddr ta(lane, C::RB, C::SWM);
    const int i0 = zs * i_per_split, i1 = min(N, i0 + i_per_split);
    const int nvg = min(64, N - g0);
    const uint64_t gvalid = nvg == 64 ? ~0ull : (1ull << nvg) - 1ull;   // the group's blocks below N

    auto dma_block = [&](int i, unsigned char* tqo, f32x4_t* trs) {
        const int rows = min(kBlock, T - i * kBlock);
        tile_dma<D>(tqo, brsrc(q + base + (int64_t)i * kBlock * D, (uint32_t)(rows * C::RB)), wave, lane);
        tile_dma<D>(tqo + C::TILE, brsrc(dout + base + (int64_t)i * kBlock * D, (uint32_t)(rows * C::RB)), wave, lane);
        if (wave == 0)   // (lse, delta, beta) of the block's rows; rows past T read zero
            dma16(brsrc(rowstat + bh * (int64_t)T + (int64_t)i * kBlock, (uint32_t)(rows * 16)), trs,
                  (uint32_t)(16 * lane));
    };

    // this lane's block as hi + lo bf16 operands (rows of kbar and V-hat, dims 16 ks + 8 g ..)
    uint4 kh[C::KS], kl[C::KS], vh[C::KS], vl[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const int64_t a = (bh * N + jc) * (int64_t)D + 16 * ks + 8 * g;
        uint32_t w[4][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float k0 = jvalid ? (float)kbar[a + 2 * e] : 0.f, k1 = jvalid ? (float)kbar[a + 2 * e + 1] : 0.f;
            const float v0 = jvalid ? vsum[a + 2 * e] : 0.f, v1 = jvalid ? vsum[a + 2 * e + 1] : 0.f;
            w[0][e] = pack_bf16x2(k0, k1);
            w[1][e] = pack_bf16x2(k0 - bf16_lo(w[0][e]), k1 - bf16_hi(w[0][e]));
            w[2][e] = pack_bf16x2(v0, v1);
            w[3][e] = pack_bf16x2(v0 - bf16_lo(w[2][e]), v1 - bf16_hi(w[2][e]));
        }
        kh[ks] = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
        kl[ks] = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
        vh[ks] = make_uint4(w[2][0], w[2][1], w[2][2], w[2][3]);
        vl[ks] = make_uint4(w[3][0], w[3][1], w[3][2], w[3][3]);
    }
    f32x16_t dka[C::DT], dva[C::DT];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) dka[dt] = dva[dt] = zero16();
    if (i0 < i1) dma_block(i0, tqo0, trs0);

    // query block i, its tiles in the arrays of parity PAR
    auto body = [&](auto par, int i) {
        constexpr int PAR = decltype(par)::value;
        unsigned char* sQ = PAR == 0 ? tqo0 : tqo1;
        unsigned char* sO = sQ + C::TILE;
        const f32x4_t* srs = PAR == 0 ? trs0 : trs1;
        // selection bits of the group's 64 blocks for query block i (scalar loads)
        const uint32_t* mrow = mask + (bh * N + i) * (int64_t)NW;
        const int wi = g0 >> 5;
        const uint64_t sel = (uint64_t)mrow[wi] | ((uint64_t)(wi + 1 < NW ? mrow[wi + 1] : 0u) << 32);
        const bool use = jvalid && !((sel >> (j - g0)) & 1ull);
        const bool any = (~sel & gvalid) != 0ull;   // uniform: some block of the group is virtual for i
        const float wg = (second_order && use) ? wgate[(bh * N + i) * (int64_t)N + j] : 0.f;
        float bias = wg * kLog2e;
        // this wave's DMAs of block i have landed; after the barrier every
        // wave's have, and every wave is done with the other parity's arrays.
        // (bias is an operand, so that its load is waited for here and not
        // after the next block's DMA, which a later wait would include.)
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : "+v"(bias) : : "memory");
        if (i + 1 < i1) dma_block(i + 1, PAR == 0 ? tqo1 : tqo0, PAR == 0 ? trs1 : trs0);
        if (!any) {   // every block of the group exact for i: no virtual pair
            if (second_order && qt == 0 && g == 0 && jvalid) dw[(bh * N + i) * (int64_t)N + j] = 0.f;
            return;
        }
        const int rows = min(kBlock, T - i * kBlock);
        f32x16_t s = zero16(), gv = zero16();
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const bf16x8_t aq = row_op<D>(sQ, qt * 32 + r32, ks, g);
            const bf16x8_t ao = row_op<D>(sO, qt * 32 + r32, ks, g);
            s = mfma(aq, as_bf16x8(kh[ks]), s);
            s = mfma(aq, as_bf16x8(kl[ks]), s);
            gv = mfma(ao, as_bf16x8(vh[ks]), gv);
            gv = mfma(ao, as_bf16x8(vl[ks]), gv);
        }
        f32x16_t a;
        float dws = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int qq = qt * 32 + acc_row(r, g);
            const f32x4_t rs = srs[qq];   // (lse, delta, beta)
            a[r] = (use && qq < rows) ? fexp2(fmaf(s[r], c2, bias - rs[0] * kLog2e)) : 0.f;
            s[r] = a[r] * (gv[r] + nj * (rs[2] - rs[1]));   // dlam
            dws += s[r];
        }
        if (second_order) {   // dW_ij: this lane's 16 rows, the other lane half, the other query half
            dws += __shfl_xor(dws, 32);
            if (qt == 1 && g == 0) sdw[kt][r32] = dws;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8_t dh, dlo, ah, alo;
            split_op(s, h, dh, dlo);
            split_op(a, h, ah, alo);
            const int r0 = qt * 32 + 16 * h;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const bf16x8_t aq = tr_op<D>(sQ, ta, dt, r0);   // Q^T dlam
                dka[dt] = mfma(aq, dh, dka[dt]);
                dka[dt] = mfma(aq, dlo, dka[dt]);
                const bf16x8_t ao = tr_op<D>(sO, ta, dt, r0);   // dO^T A
                dva[dt] = mfma(ao, ah, dva[dt]);
                dva[dt] = mfma(ao, alo, dva[dt]);
            }
        }
        if (second_order) {
            // LDS writes done, then the barrier (no wait for the DMA in flight)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (qt == 0 && g == 0 && jvalid)
                dw[(bh * N + i) * (int64_t)N + j] = wg != 0.f ? dws + sdw[kt][r32] : 0.f;
        }
    };
    for (int i = i0; i < i1; i += 2) {
        body(std::integral_constant<int, 0>(), i);
        if (i + 1 < i1) body(std::integral_constant<int, 1>(), i + 1);
    }
    // the two query halves of each block tile: wave (kt, 1) hands its partials to wave (kt, 0)
    float* xs = reinterpret_cast<float*>(tqo0);
    const int64_t pbase = ((int64_t)zs * gridDim.y + bh) * N * (int64_t)D;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        f32x16_t* acc = pass == 0 ? dva : dka;
        __syncthreads();
        if (qt == 1) {
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xs[((kt * C::DT + dt) * 16 + r) * 64 + lane] = acc[dt][r];
        }
        __syncthreads();
        if (qt == 0 && jvalid) {
            float* out = (pass == 0 ? dvh_part : dkb_part) + pbase + (int64_t)j * D;
            const float sc = pass == 0 ? 1.f : scale;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int run = 0; run < 4; ++run) {
                    f32x4_t w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * run + e;
                        w[e] = sc * (acc[dt][r] + xs[((kt * C::DT + dt) * 16 + r) * 64 + lane]);
                    }
                    *reinterpret_cast<f32x4_t*>(out + dt * 32 + 8 * run + 4 * g) = w;
                }
        }
    }
}

// dsig2_j = 1/2 sum_i dW_ij q2bar_i (dW is 0 for gated and exact pairs).
__global__ __launch_bounds__(128) void bwd_dsig2_kernel(const float* __restrict__ dw, const double* __restrict__ q2bar,
                                                        float* __restrict__ dsg, int N, int D) {
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    for (int d = threadIdx.x; d < D; d += 128) {
        float acc = 0.f;
        for (int i = 0; i < N; ++i) acc = fmaf(dw[(bh * N + i) * (int64_t)N + j], (float)q2bar[(bh * N + i) * (int64_t)D + d], acc);
        dsg[(bh * N + j) * (int64_t)D + d] = 0.5f * acc;
    }
}

}  // namespace

int bwd_virt_splits(const Geom& g) {
    const int64_t groups = (int64_t)((g.N + 63) / 64) * g.BH;
    int s = (int)((1024 + groups - 1) / groups);
    return s < 1 ? 1 : (s > 8 ? 8 : (s > g.N ? g.N : s));
}

hipError_t launch_bwd_virt_mfma(const Geom& g, const bf16_t* q, const bf16_t* dout, const StatsView* st,
                                const uint32_t* mask, const f32x4_t* rowstat, const float* wgate, float* dkb_part,
                                float* dvh_part, float* dw, float* dsg, int NW, int second_order,
                                hipStream_t stream) {
    const int S = bwd_virt_splits(g);
    const int per = (g.N + S - 1) / S;
    const dim3 grid((g.N + 63) / 64, (unsigned)g.BH, S);
    if (g.D == 128)
        hipLaunchKernelGGL((bwd_virt_mfma_kernel<128>), grid, dim3(kThreads), 0, stream, q, dout, st->kbar, st->vsum,
                           mask, rowstat, wgate, dkb_part, dvh_part, dw, g.T, g.N, NW, g.scale, second_order, per);
    else
        hipLaunchKernelGGL((bwd_virt_mfma_kernel<64>), grid, dim3(kThreads), 0, stream, q, dout, st->kbar, st->vsum,
                           mask, rowstat, wgate, dkb_part, dvh_part, dw, g.T, g.N, NW, g.scale, second_order, per);
    if (second_order)
        hipLaunchKernelGGL(bwd_dsig2_kernel, dim3(g.N, (unsigned)g.BH), dim3(128), 0, stream, dw, st->q2bar, dsg,
                           g.N, g.D);
    return hipGetLastError();
}

hipError_t launch_bwd_prep(const Geom& g, const StatsView* st, bf16_t* kbh, bf16_t* kbl, bf16_t* vhh,
                           bf16_t* vhl, bf16_t* hh, bf16_t* hl, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_prep_kernel, dim3(g.N + 1, (unsigned)g.BH), dim3(kThreads), 0, stream, st->kbar, st->vsum,
                       st->hsum, kbh, kbl, vhh, vhl, hh, hl, g.N, g.D);
    return hipGetLastError();
}

hipError_t launch_bwd_rowstats(const Geom& g, const bf16_t* q, const bf16_t* k, const bf16_t* o, const bf16_t* dout,
                               const bf16_t* kbh, const bf16_t* kbl, const bf16_t* hh, const bf16_t* hl,
                               const uint32_t* mask, const float* wgate, f32x4_t* rowstat, int NW, int second_order,
                               int first_order, hipStream_t stream) {
    const dim3 grid(g.N, (unsigned)g.BH);
#define PISA_ROWSTATS(DD)                                                                                      \
    hipLaunchKernelGGL((bwd_rowstats_kernel<DD>), grid, dim3(kThreads), 0, stream, q, k, o, dout, kbh, kbl, hh, \
                       hl, mask, wgate, rowstat, g.T, g.N, NW, g.scale, second_order, first_order)
    if (g.D == 128) PISA_ROWSTATS(128);
    else PISA_ROWSTATS(64);
#undef PISA_ROWSTATS
    return hipGetLastError();
}

hipError_t launch_bwd_rowstats_fwd(const Geom& g, const bf16_t* q, const bf16_t* o, const bf16_t* dout,
                                   const bf16_t* hh, const bf16_t* hl, const float* fwd_rstat, f32x4_t* rowstat,
                                   int first_order, hipStream_t stream) {
    const dim3 grid((g.N + kRsBlocks - 1) / kRsBlocks, (unsigned)g.BH);
    if (g.D == 128)
        hipLaunchKernelGGL((bwd_rowstats_fwd_kernel<128>), grid, dim3(kThreads), 0, stream, q, o, dout, hh, hl,
                           fwd_rstat, rowstat, g.T, g.N, g.scale, first_order);
    else
        hipLaunchKernelGGL((bwd_rowstats_fwd_kernel<64>), grid, dim3(kThreads), 0, stream, q, o, dout, hh, hl,
                           fwd_rstat, rowstat, g.T, g.N, g.scale, first_order);
    return hipGetLastError();
}

hipError_t launch_bwd_dh_mfma(const Geom& g, const bf16_t* q, const bf16_t* dout, const f32x4_t* rowstat,
                              float* part, int parts, hipStream_t stream) {
    const int rows_per = (g.T + parts - 1) / parts;
    const dim3 grid((unsigned)parts, (unsigned)g.BH);
    if (g.D == 128)
        hipLaunchKernelGGL((bwd_dh_mfma_kernel<128>), grid, dim3(kThreads), 0, stream, q, dout, rowstat, part, g.T,
                           rows_per, g.scale);
    else
        hipLaunchKernelGGL((bwd_dh_mfma_kernel<64>), grid, dim3(kThreads), 0, stream, q, dout, rowstat, part, g.T,
                           rows_per, g.scale);
    return hipGetLastError();
}

hipError_t launch_bwd_dq(const Geom& g, const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* dout,
                         const bf16_t* kbh, const bf16_t* kbl, const bf16_t* vhh, const bf16_t* vhl,
                         const bf16_t* hh, const bf16_t* hl, const uint32_t* mask, const float* wgate,
                         const f32x4_t* rowstat, const float* dw, const double* ksig2, float* dq2, bf16_t* dq, int NW,
                         int second_order, int first_order, hipStream_t stream) {
    const dim3 grid(g.N, (unsigned)g.BH);
    if (second_order)
        hipLaunchKernelGGL(bwd_dq2_kernel, grid, dim3(128), 0, stream, dw, ksig2, dq2, g.N, g.D);
#define PISA_DQ(DD)                                                                                            \
    hipLaunchKernelGGL((bwd_dq_kernel<DD>), grid, dim3(kThreads), 0, stream, q, k, v, dout, kbh, kbl, vhh, vhl, \
                       hh, hl, mask, wgate, rowstat, dq2, dq, g.T, g.N, NW, g.scale, second_order, first_order)
    if (g.D == 128) PISA_DQ(128);
    else PISA_DQ(64);
#undef PISA_DQ
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const Geom& g, const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* dout,
                           const uint32_t* mask, const f32x4_t* rowstat, const StatsView* st, const float* dH,
                           const float* dHT, const float* dkb_part, const float* dvh_part, const float* dsg,
                           bf16_t* dk, bf16_t* dv, int NW, int nsplit, int second_order, int first_order,
                           hipStream_t stream) {
    const dim3 grid(g.N, (unsigned)g.BH);
#define PISA_DKDV(DD)                                                                                          \
    hipLaunchKernelGGL((bwd_dkdv_exact_kernel<DD>), grid, dim3(kThreads), 0, stream, q, k, v, dout, mask, rowstat, \
                       st->kbar, st->vsum, dH, dHT, dkb_part, dvh_part, dsg, dk, dv, g.T, g.N, NW, g.scale, nsplit, \
                       second_order, first_order)
    if (g.D == 128) PISA_DKDV(128);
    else PISA_DKDV(64);
#undef PISA_DKDV
    return hipGetLastError();
}

}  // namespace pisa
