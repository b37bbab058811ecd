// Internal declarations shared by the libpisa translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa.h"

namespace pisa {

constexpr int kBlock = 64;        // rows per query / KV block (the paper's 64x64 kernel block)
constexpr int kThreads = 256;     // workgroup size of every kernel (4 wave64)

typedef unsigned short bf16_t;    // bf16 storage (bit pattern)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T> __device__ __forceinline__ T store_cast(float x);
template <> __device__ __forceinline__ float store_cast<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t store_cast<bf16_t>(float x) { return f32_to_bf16(x); }

// The forced exact set of query block i: the band [lo, hi] = [i - band,
// i + band] clipped to [0, N), then the sink blocks [0, ns) outside it.
// forced_count gives its size, forced_block(c) its c-th member (band blocks
// ascending, then the sinks below lo, then those above hi).
struct Forced {
    int lo, hi, ns;
    __host__ __device__ Forced(int i, int band, int n_sink, int N)
        : lo(i - band > 0 ? i - band : 0), hi(i + band < N - 1 ? i + band : N - 1),
          ns(n_sink < N ? n_sink : N) {}
    __host__ __device__ int below() const { return ns < lo ? ns : lo; }
    __host__ __device__ int above() const { return ns - hi - 1 > 0 ? ns - hi - 1 : 0; }
    __host__ __device__ int count() const { return hi - lo + 1 + below() + above(); }
    __host__ __device__ int block(int c) const {
        const int nb = hi - lo + 1;
        if (c < nb) return lo + c;
        c -= nb;
        return c < below() ? c : hi + 1 + (c - below());
    }
    __host__ __device__ bool forced(int j) const { return (j >= lo && j <= hi) || j < ns; }
};

// The tile (x, y, z) of this workgroup in its grid, XCD-aware: workgroups are
// dispatched in linear order (x fastest) and dealt round-robin to the 8 XCDs,
// so consecutive ids land on different XCDs; this bijection of the linear ids
// gives each XCD a contiguous range of tiles instead, so that neighbouring
// tiles (blocks of one head, whose operands overlap) share that XCD's L2.
__device__ __forceinline__ void xcd_tile(int* x, int64_t* y, int* z = nullptr) {
    const int64_t nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
    const int64_t lin = ((int64_t)blockIdx.z * ny + blockIdx.y) * nx + blockIdx.x;
    const int64_t xcd = lin % 8, pos = lin / 8, per = total / 8, rem = total % 8;
    const int64_t L = xcd < rem ? xcd * (per + 1) + pos : rem * (per + 1) + (xcd - rem) * per + pos;
    *x = (int)(L % nx);
    *y = (L / nx) % ny;
    if (z) *z = (int)(L / (nx * ny));
}

// What the kernels read and write: the caller's statistics (pisa_stats_t)
// and the views of its operand buffer (the kernels' own layouts of them).
struct StatsView {
    double* qbar;
    double* q2bar;
    double* kbar;
    float* vsum;
    double* ksig2;
    float* hsum;
    double* hnorm;     // ||H_j - Hbar||_F per block (covariance prior)  [BH,N]
    void* kbar_c;      // kbar rounded to the input dtype              [BH,N,D]
    void* vbar_c;      // vsum / n rounded to the input dtype          [BH,N,D]
    void* kpack;       // bf16: K in the fused kernel's operand order  [BH,N,64 D]
    void* hpack;       // bf16: H split hi + lo, operand order         [BH,2 D D]
    void* kbpack;      // bf16: kbar_c in kpack's order per 64 blocks  [BH,ceil(N/64),64 D]
    bf16_t* kbar_r;    // kbar split bf16 hi + lo, the router's operand order [BH,ceil(N/16) 16 D 2]
    bf16_t* ksig2_r;   // ksig2 the same way
    float* knorm;      // ||kbar_j||_2 rounded up (the router's error bound) [BH,ceil(N/16) 16]
};

// The router's operand order for a per-block row x[j][d] (kbar or ksig2) of a
// head: split into bf16 hi = rn(x), lo = rn(x - hi) (|x - hi - lo| <= 2^-17 |x|),
// chunk c = j / 16 of 16 keys, k-step s < D / 32, part p (hi, lo), lane
// 16 g + (j % 16) with d = (D / 4) g + 8 s + e: bf16 element
// ((c D/32 + s) 2 + p) 512 + (16 g + j % 16) 8 + e. A 64-lane 16-byte load of
// (c, s, p) is one MFMA 16x16x32 B operand of 16 keys.
__device__ __forceinline__ void router_store(bf16_t* head, int j, int d, int D, double x) {
    const int c = j >> 4, n16 = j & 15, g = d / (D / 4), s = (d % (D / 4)) >> 3, e = d & 7;
    const int64_t o = (int64_t)((c * (D / 32) + s) * 2) * 512 + (16 * g + n16) * 8 + e;
    const bf16_t hi = f32_to_bf16((float)x);
    head[o] = hi;
    head[o + 512] = f32_to_bf16((float)(x - (double)bf16_to_f32(hi)));
}
__host__ __device__ inline int64_t router_head_elems(int N, int D) { return (int64_t)((N + 15) / 16) * 16 * D * 2; }

// Problem geometry resolved once on the host.
struct Geom {
    int64_t BH;       // batch * heads
    int T;            // tokens
    int D;            // head dim
    int N;            // blocks
    float scale;      // softmax scale (fp32)
    double scale64;   // the same scale in fp64 (routing decisions)
};

// Byte offsets of the kernel layouts inside a caller's operand buffer (each
// 256-byte aligned; the bf16-only layouts are empty for fp32 inputs), in the
// order of pisa_operand_t, and the buffer's total size.
struct OperandLayout {
    size_t off[PISA_OPERAND_COUNT];
    size_t bytes[PISA_OPERAND_COUNT];
    size_t total;
};
OperandLayout operand_layout(const Geom& g, int dtype);
// The kernel view of caller statistics plus an operand buffer.
StatsView stats_view(const Geom& g, int dtype, const pisa_stats_t* st, const void* operands);

// Kernel launchers (return hipSuccess or the launch error).
hipError_t launch_block_stats(const Geom& g, int dtype, int second_order, int cov_bias, const void* q,
                              const void* k, const void* v, const StatsView* out, void* workspace,
                              hipStream_t stream);
// Workspace of pisa_block_stats: the larger of its two uses (fp32 partial H
// sums; with the covariance prior, fp64 partial sums and Hbar).
size_t stats_workspace_bytes(const Geom& g);
size_t stats_workspace_bytes_for(const Geom& g, int cov_bias);
size_t cov_workspace_bytes(const Geom& g, int stats_groups);
hipError_t launch_cov_norm(const Geom& g, int dtype, const void* k, const void* v, const double* kbar,
                           double* hnorm, void* workspace, int stats_groups, hipStream_t stream);
// This device's copy of the statistics pass's static scratch
// (PISA_STATS_SCRATCH_BYTES), its address taken once per device.
hipError_t stats_scratch(void** ptr);
// The operand layouts from statistics of any source (and K for kpack).
hipError_t launch_prepare_operands(const Geom& g, int dtype, int second_order, const void* k,
                                   const StatsView* st, hipStream_t stream);

hipError_t launch_route_topk(const Geom& g, const pisa_params_t* p, const StatsView* st,
                             int32_t* idx, float* wgate, hipStream_t stream);

hipError_t launch_attn_fwd_valu(const Geom& g, int dtype, const pisa_params_t* p, const void* q,
                                const void* k, const void* v, const StatsView* st,
                                const int32_t* idx, const float* wgate, void* o, float* rstat,
                                hipStream_t stream);

// fp32 inputs on the fp32 matrix cores (reads stats kbar, vsum, hsum).
hipError_t launch_attn_fwd_f32(const Geom& g, const pisa_params_t* p, const void* q, const void* k,
                               const void* v, const StatsView* st, const int32_t* idx, const float* wgate,
                               void* o, float* rstat, hipStream_t stream);

hipError_t launch_reorder(const Geom& g, int64_t batch, int64_t heads, int elem_bytes, bool gather,
                          const int32_t* perm, const void* src, void* dst, hipStream_t stream);
void z_order_host(const int64_t* grid, int ndim, int64_t prefix, int32_t* perm);

size_t attn_bwd_workspace_bytes(const Geom& g, int dtype);
hipError_t launch_bwd_prep(const Geom& g, const StatsView* st, bf16_t* kbh, bf16_t* kbl, bf16_t* vhh,
                           bf16_t* vhl, bf16_t* hh, bf16_t* hl, hipStream_t stream);
hipError_t launch_bwd_rowstats(const Geom& g, const bf16_t* q, const bf16_t* k, const bf16_t* o, const bf16_t* dout,
                               const bf16_t* kbh, const bf16_t* kbl, const bf16_t* hh, const bf16_t* hl,
                               const uint32_t* mask, const float* wgate, f32x4_t* rowstat, int NW, int second_order,
                               int first_order, hipStream_t stream);
// Row statistics from the forward's per-row lse and c: only delta and beta computed.
hipError_t launch_bwd_rowstats_fwd(const Geom& g, const bf16_t* q, const bf16_t* o, const bf16_t* dout,
                                   const bf16_t* hh, const bf16_t* hl, const float* fwd_rstat, f32x4_t* rowstat,
                                   int first_order, hipStream_t stream);
// dH partial sums over `parts` row ranges on the matrix cores (bf16 inputs).
hipError_t launch_bwd_dh_mfma(const Geom& g, const bf16_t* q, const bf16_t* dout, const f32x4_t* rowstat,
                              float* part, int parts, hipStream_t stream);
hipError_t launch_bwd_dq(const Geom& g, const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* dout,
                         const bf16_t* kbh, const bf16_t* kbl, const bf16_t* vhh, const bf16_t* vhl,
                         const bf16_t* hh, const bf16_t* hl, const uint32_t* mask, const float* wgate,
                         const f32x4_t* rowstat, const float* dw, const double* ksig2, float* dq2, bf16_t* dq, int NW,
                         int second_order, int first_order, hipStream_t stream);
int bwd_virt_splits(const Geom& g);
hipError_t launch_bwd_virt_mfma(const Geom& g, const bf16_t* q, const bf16_t* dout, const StatsView* st,
                                const uint32_t* mask, const f32x4_t* rowstat, const float* wgate, float* dkb_part,
                                float* dvh_part, float* dw, float* dsg, int NW, int second_order,
                                hipStream_t stream);
hipError_t launch_bwd_dkdv(const Geom& g, const bf16_t* q, const bf16_t* k, const bf16_t* v, const bf16_t* dout,
                           const uint32_t* mask, const f32x4_t* rowstat, const StatsView* st, const float* dH,
                           const float* dHT, const float* dkb_part, const float* dvh_part, const float* dsg,
                           bf16_t* dk, bf16_t* dv, int NW, int nsplit, int second_order, int first_order,
                           hipStream_t stream);
hipError_t launch_attn_bwd(const Geom& g, int dtype, const pisa_params_t* p, const void* q, const void* k,
                           const void* v, const void* o, const void* dout, const StatsView* st,
                           const int32_t* idx, const float* wgate, const float* fwd_rstat, void* dq, void* dk,
                           void* dv, void* ws, hipStream_t stream);

// Kernel choice of pisa_attn_fwd (a pisa_attn_kernel_t) and the longest
// per-wave item list of the persistent bf16 kernel for these parameters.
int64_t attn_asm_wave_items(const Geom& g, const pisa_params_t* p);
int attn_fwd_kernel(const Geom& g, int dtype, const pisa_params_t* p);

hipError_t launch_attn_fwd_mfma(const Geom& g, const pisa_params_t* p, const void* q, const void* k,
                                const void* v, const StatsView* st, const int32_t* idx,
                                const float* wgate, void* o, float* rstat, hipStream_t stream);

}  // namespace pisa
