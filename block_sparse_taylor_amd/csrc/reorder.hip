// Morton (Z-order) token reorder around the operator ("Piecewise-Taylor-
// Attention" README: the Wan2.1 results paragraph, 64-token blocks over a
// Z-order tile reordering of the latent grid, and the changelog item on the
// Morton tile reorder with its fused gather kernel): one pass that gathers the
// tokens into the new order while transposing [B,T,H,D] into the operator's
// [B,H,T,D], and its inverse on the output.
//
// The permutation itself is host work done once per grid (pisa_z_order): a
// cell's code interleaves the bits of its coordinates, the fastest axis on the
// lowest bit of every bit group, and cells are visited in ascending code.
//
// The kernels are pure HBM streams. A workgroup owns TT consecutive positions
// i of one batch entry and moves every head of them: 16-byte chunks ordered
// (position, head, chunk) with the chunk fastest, so that the token-major
// side is one contiguous run of H * D * e bytes per token and the head-major
// side one run of D * e bytes per (head, position), 16 lanes wide. Each lane
// issues kUnroll loads before its stores; both are non-temporal (every byte is
// touched once), and a workgroup moves 32 KB: about 5.2 TB/s at the Wan2.1
// shape, against 5.4-5.5 TB/s for a plain device copy of the same bytes.
#include <algorithm>
#include <numeric>
#include <vector>

#include "common.h"

namespace pisa {
namespace {

constexpr int kUnroll = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kChunksPerGroup = 2048;   // 16-byte chunks a workgroup moves (32 KB)

template <bool kGather>
__global__ __launch_bounds__(kThreads) void reorder_kernel(const uint4* __restrict__ src,
                                                           uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ perm, int T,
                                                           int H, int CH, int TT) {
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.y;
    const int i0 = blockIdx.x * TT;
    const int nt = min(TT, T - i0);
    const int per_tok = H * CH;
    const int total = nt * per_tok;
    for (int c0 = 0; c0 < total; c0 += kThreads * kUnroll) {
        u32x4 val[kUnroll];
        int64_t to[kUnroll];
        bool st[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = c0 + u * kThreads + tid;
            const bool in = c < total;
            const int r = in ? c / per_tok : 0;
            const int rem = c - r * per_tok;
            const int h = rem / CH, ch = rem - h * CH;
            const int i = i0 + r;
            const int t = in ? perm[i] : -1;
            const bool ok = t >= 0 && t < T;
            const int64_t tok = ((b * T + t) * H + h) * CH + ch;   // [B,T,H,D] chunk of token t
            const int64_t hm = ((b * H + h) * T + i) * CH + ch;    // [B,H,T,D] chunk of position i
            if (kGather) {
                val[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + tok) : (u32x4){0u, 0u, 0u, 0u};
                to[u] = hm;
                st[u] = in;
            } else {
                val[u] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + hm) : (u32x4){0u, 0u, 0u, 0u};
                to[u] = tok;
                st[u] = ok;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (st[u]) __builtin_nontemporal_store(val[u], reinterpret_cast<u32x4*>(dst) + to[u]);
    }
}

}  // namespace

hipError_t launch_reorder(const Geom& g, int64_t batch, int64_t heads, int elem_bytes, bool gather,
                          const int32_t* perm, const void* src, void* dst, hipStream_t stream) {
    const int CH = g.D * elem_bytes / 16;
    const int per_tok = (int)heads * CH;
    const int TT = std::max(1, std::min(kBlock * 4, kChunksPerGroup / per_tok));
    const dim3 grid((unsigned)((g.T + TT - 1) / TT), (unsigned)batch), block(kThreads);
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    if (gather)
        hipLaunchKernelGGL(reorder_kernel<true>, grid, block, 0, stream, s, d, perm, g.T, (int)heads, CH, TT);
    else
        hipLaunchKernelGGL(reorder_kernel<false>, grid, block, 0, stream, s, d, perm, g.T, (int)heads, CH, TT);
    return hipGetLastError();
}

void z_order_host(const int64_t* grid, int ndim, int64_t prefix, int32_t* perm) {
    int nb = 1;
    for (int a = 0; a < ndim; ++a)
        while ((int64_t{1} << nb) < grid[a]) ++nb;
    int64_t cells = 1;
    for (int a = 0; a < ndim; ++a) cells *= grid[a];
    std::vector<uint64_t> code((size_t)cells);
    std::vector<int64_t> coord((size_t)ndim);
    for (int64_t r = 0; r < cells; ++r) {
        int64_t x = r;   // raster index -> coordinates, fastest axis last
        for (int a = ndim - 1; a >= 0; --a) {
            coord[a] = x % grid[a];
            x /= grid[a];
        }
        uint64_t z = 0;
        for (int bit = 0; bit < nb; ++bit)
            for (int slot = 0; slot < ndim; ++slot)   // slot 0: the fastest axis
                z |= (uint64_t)((coord[ndim - 1 - slot] >> bit) & 1) << (ndim * bit + slot);
        code[(size_t)r] = z;
    }
    std::vector<int64_t> order((size_t)cells);
    std::iota(order.begin(), order.end(), int64_t{0});
    std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return code[(size_t)a] < code[(size_t)b]; });
    for (int64_t i = 0; i < prefix; ++i) perm[i] = (int32_t)i;
    for (int64_t i = 0; i < cells; ++i) perm[prefix + i] = (int32_t)(prefix + order[(size_t)i]);
}

}  // namespace pisa
