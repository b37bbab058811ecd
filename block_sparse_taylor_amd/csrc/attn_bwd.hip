// Backward of the fused PISA forward: dq, dk, dv of L = sum_t dout_t . o_t
// with the routing table and the second-order gate held constant
// (Piecewise-Taylor-Attention README: the trainable regime, a backward pass
// through both branches with the selection detached; PISA §3.2 Eqs. 3-5 and
// §3.3 Eqs. 9-10 for the forward it differentiates). This file holds the
// fp32-input kernels (VALU, fp32 arithmetic) and the mask, dH and chain
// kernels both dtypes share; bf16 inputs run every product on the matrix
// cores (attn_bwd_mfma.hip). Results in the input dtype.
//
// Per query row t of block i, with q' = s q_t, g = dout_t, den_t the
// normaliser, lse_t = log den_t, l_t the tail mass and T the sequence length:
//   exact key k (block in S_i): P = e^{q'.k - lse},  dz = P (g.v - delta),
//   virtual token j (in U_i):   A = e^{lam - lse},   dlam = A (g.V-hat_j + n_j (beta - delta)),
//   delta = g . o_t,  beta = g . (q' H) / T,  c_t = l_t / (T den_t).
// Gradients:
//   dq'  = sum_exact dz k + sum_virtual dlam kbar_j + c_t H g,
//   dk   = sum_t dz q'  (+ chain),            dv = sum_t P g (+ chain),
//   dkbar_j = sum_t dlam q' - dH V-hat_j,     dV-hat_j = sum_t A g,
//   dH   = sum_t c_t q' g^T,
//   and for the gated second-order logit w_ij = 1/2 q2bar_i . sig2_j:
//   dW_ij = sum_{t in i} dlam_tj,  dq2bar_i = 1/2 sum_j dW_ij sig2_j,
//   dsig2_j = 1/2 sum_i dW_ij q2bar_i (over kept pairs only).
// The chain to the tokens: kbar_j is a mean (dk += dkbar_j / n_j), V-hat_j a
// sum (dv += dV-hat_j), H = sum (k - kbar)^T v (dk += dH v, dv += dH^T (k - kbar)),
// sig2_j a mean square (dk += 2 dsig2_j (k - kbar_j) / n_j), q2bar_i a mean
// square of q' (dq += 2 s q' dq2bar_i / n_i).
// A gated pair stores w = 0 in wgate; a kept pair with w = 0 has q2bar_i
// sig2_j = 0 in every dimension, where both chain terms vanish, so "wgate
// != 0" is the gate for the gradient.
//
// Kernels (all deterministic: fixed loop orders, no floating-point atomics):
//   mask  - bit j of row i set iff block j is exact for query block i,
//   row   - per query block: lse, delta, beta, c (rowstat) and dq (fp32),
//   dh    - partial sums of dH over row chunks, then their fixed-order sum,
//   virt  - per group of 16 KV blocks: dkbar (virtual part), dV-hat, dsig2 (fp32),
//   kv    - per KV block: dk, dv of the exact pairs plus every chain term
//           (fp32; for bf16 the matrix-core dk/dv kernel does both).
#include <math.h>

#include <type_traits>

#include "common.h"

namespace pisa {
namespace {

constexpr int kSub = 32;          // K/V rows staged per step in the row kernel
constexpr int kRowThreads = 128;  // row kernel: 2 threads per query row
constexpr int kVirtBlocks = 16;   // KV blocks per virt workgroup (4 threads each)
constexpr int kVirtRows = 16;     // query rows staged per step in the virt kernel
constexpr int kKvRows = 64;       // query rows staged per step in the kv kernel
constexpr int kDhMaxParts = 64;   // row chunks of the dH partial sums

__device__ __forceinline__ bool bit_set(const uint32_t* w, int j) { return (w[j >> 5] >> (j & 31)) & 1u; }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

__device__ __forceinline__ f32x4_t lds4(const float* p) { return *reinterpret_cast<const f32x4_t*>(p); }

int dh_parts(int T) {
    const int p = (T + 511) / 512;
    return p < 1 ? 1 : (p > kDhMaxParts ? kDhMaxParts : p);
}

// ---------------------------------------------------------------- mask
__global__ __launch_bounds__(64) void bwd_mask_kernel(const int32_t* __restrict__ idx, uint32_t* __restrict__ mask,
                                                      int N, int NW, int topk, int band, int n_sink) {
    extern __shared__ uint32_t words[];
    const int i = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const Forced fs(i, band, n_sink, N);
    for (int w = threadIdx.x; w < NW; w += 64) {
        uint32_t b = 0;
        for (int e = 0; e < 32; ++e) {
            const int j = 32 * w + e;
            if (j < N && fs.forced(j)) b |= 1u << e;
        }
        words[w] = b;
    }
    __syncthreads();
    if (idx && topk > 0) {
        const int32_t* row = idx + (bh * N + i) * (int64_t)topk;
        for (int c = threadIdx.x; c < topk; c += 64) {
            const int j = row[c];
            if (j >= 0 && j < N) atomicOr(&words[j >> 5], 1u << (j & 31));   // integer OR: order-free
        }
    }
    __syncthreads();
    uint32_t* out = mask + (bh * N + i) * (int64_t)NW;
    for (int w = threadIdx.x; w < NW; w += 64) out[w] = words[w];
}

// ---------------------------------------------------------------- row
// One workgroup of 128 threads per (bh, query block i); threads 2r and 2r+1
// share query row r, thread h owning dims 8c + 4h + e (c < D/8, e < 4).
template <typename T, int D>
__global__ __launch_bounds__(kRowThreads) void bwd_row_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ o,
    const T* __restrict__ dout, const double* __restrict__ kbar, const float* __restrict__ vsum,
    const double* __restrict__ ksig2, const float* __restrict__ hsum, const uint32_t* __restrict__ mask,
    const float* __restrict__ wgate, T* __restrict__ dq, f32x4_t* __restrict__ rowstat, int Tn, int N, int NW,
    float scale, int second_order, int first_order) {
    constexpr int C = D / 8;
    constexpr int HD = D / 2;
    constexpr int DPL = D / 64;     // dq2bar dims per lane of a wave
    __shared__ __attribute__((aligned(16))) float sk[kSub * D];
    __shared__ __attribute__((aligned(16))) float sv[kSub * D];
    __shared__ float sdq2[2][D];
    extern __shared__ uint32_t sel[];

    const int tid = threadIdx.x;
    const int r = tid >> 1, h = tid & 1, lane = tid & 63, wave = tid >> 6;
    const int64_t bh = blockIdx.y;
    const int i = blockIdx.x;
    const int r0 = i * kBlock;
    const int rows = min(kBlock, Tn - r0);
    const int t = r0 + r;
    const bool active = r < rows;
    const int64_t base = bh * (int64_t)Tn * D;

    float qv[HD], g[HD], dqv[HD];
    float delta = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 8 * c + 4 * h + e;
            const int64_t a = base + (int64_t)t * D + d;
            qv[4 * c + e] = active ? load_f32(q + a) * scale : 0.f;
            g[4 * c + e] = active ? load_f32(dout + a) : 0.f;
            if (active) delta = fmaf(g[4 * c + e], load_f32(o + a), delta);
            dqv[4 * c + e] = 0.f;
        }
    delta += __shfl_xor(delta, 1);

    for (int w = tid; w < NW; w += kRowThreads) sel[w] = mask[(bh * N + i) * (int64_t)NW + w];
    __syncthreads();

    auto dot = [&](const float* row, const float* x) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const f32x4_t kv = lds4(row + 8 * c + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) s = fmaf(x[4 * c + e], kv[e], s);
        }
        return s + __shfl_xor(s, 1);
    };

    const double* kb = kbar + bh * (int64_t)N * D;
    const float* vs = vsum + bh * (int64_t)N * D;
    const float* wr = second_order ? wgate + (bh * (int64_t)N + i) * N : nullptr;

    // Pass 1: the forward's normaliser (running max m, sum l, tail mass lt).
    float m = -INFINITY, l = 0.f, lt = 0.f;
    for (int j = 0; j < N; ++j) {
        if (!bit_set(sel, j)) continue;
        const int nj = min(kBlock, Tn - j * kBlock);
        for (int h0 = 0; h0 < nj; h0 += kSub) {
            const int nh = min(kSub, nj - h0);
            const int64_t src = base + ((int64_t)j * kBlock + h0) * D;
            __syncthreads();
            for (int c = tid; c < nh * D; c += kRowThreads) sk[c] = load_f32(k + src + c);
            __syncthreads();
            for (int n = 0; n < nh; ++n) {
                const float z = dot(sk + n * D, qv);
                if (z > m) {
                    const float cr = expf(m - z);
                    l *= cr;
                    lt *= cr;
                    m = z;
                }
                l += expf(z - m);
            }
        }
    }
    for (int j0 = 0; j0 < N; j0 += kSub) {
        const int nh = min(kSub, N - j0);
        __syncthreads();
        for (int c = tid; c < nh * D; c += kRowThreads) sk[c] = (float)kb[(int64_t)j0 * D + c];
        __syncthreads();
        for (int n = 0; n < nh; ++n) {
            const int j = j0 + n;
            if (bit_set(sel, j)) continue;
            const int nj = min(kBlock, Tn - j * kBlock);
            const float z = dot(sk + n * D, qv) + (second_order ? wr[j] : 0.f);
            const float zm = z + logf((float)nj);
            if (zm > m) {
                const float cr = expf(m - zm);
                l *= cr;
                lt *= cr;
                m = zm;
            }
            const float mass = expf(z - m) * (float)nj;
            l += mass;
            lt += mass;
        }
    }
    const float lse = m + logf(l);
    const float cf = first_order ? (lt / l) / (float)Tn : 0.f;

    // beta = g . (q' H) / T = q' . (H g) / T, and dq' starts at c_t H g.
    float beta = 0.f;
    if (first_order) {
        const float* Hm = hsum + bh * (int64_t)D * D;
#pragma unroll
        for (int d0 = 0; d0 < D; d0 += kSub) {
            __syncthreads();
            for (int c = tid; c < kSub * D; c += kRowThreads) sk[c] = Hm[(int64_t)d0 * D + c];
            __syncthreads();
#pragma unroll
            for (int dd = 0; dd < kSub; ++dd) {
                const int d = d0 + dd;
                const float hg = dot(sk + dd * D, g);   // (H g)_d
                const int y = 4 * (d >> 3) + (d & 3);
                if (((d >> 2) & 1) == h) {
                    beta = fmaf(qv[y], hg, beta);
                    dqv[y] = cf * hg;
                }
            }
        }
        beta += __shfl_xor(beta, 1);
        beta /= (float)Tn;
    }
    if (active && h == 0) {
        f32x4_t rs = {lse, delta, beta, cf};
        rowstat[bh * (int64_t)Tn + t] = rs;
    }

    // Pass 2: dq' over the exact keys.
    for (int j = 0; j < N; ++j) {
        if (!bit_set(sel, j)) continue;
        const int nj = min(kBlock, Tn - j * kBlock);
        for (int h0 = 0; h0 < nj; h0 += kSub) {
            const int nh = min(kSub, nj - h0);
            const int64_t src = base + ((int64_t)j * kBlock + h0) * D;
            __syncthreads();
            for (int c = tid; c < nh * D; c += kRowThreads) {
                sk[c] = load_f32(k + src + c);
                sv[c] = load_f32(v + src + c);
            }
            __syncthreads();
            for (int n = 0; n < nh; ++n) {
                const float z = dot(sk + n * D, qv);
                const float dp = dot(sv + n * D, g);
                const float ds = expf(z - lse) * (dp - delta);
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const f32x4_t kv = lds4(sk + n * D + 8 * c + 4 * h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dqv[4 * c + e] = fmaf(ds, kv[e], dqv[4 * c + e]);
                }
            }
        }
    }
    // ... and over the virtual tokens (with dW_ij for the second-order term).
    float dq2[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) dq2[e] = 0.f;
    const double* sg2 = second_order ? ksig2 + bh * (int64_t)N * D : nullptr;
    for (int j0 = 0; j0 < N; j0 += kSub) {
        const int nh = min(kSub, N - j0);
        __syncthreads();
        for (int c = tid; c < nh * D; c += kRowThreads) {
            sk[c] = (float)kb[(int64_t)j0 * D + c];
            sv[c] = vs[(int64_t)j0 * D + c];
        }
        __syncthreads();
        for (int n = 0; n < nh; ++n) {
            const int j = j0 + n;
            if (bit_set(sel, j)) continue;
            const int nj = min(kBlock, Tn - j * kBlock);
            const float wg = second_order ? wr[j] : 0.f;
            const float lam = dot(sk + n * D, qv) + wg;
            const float gv = dot(sv + n * D, g);
            const float a = expf(lam - lse);
            const float dl = a * (gv + (float)nj * (beta - delta));
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const f32x4_t kv = lds4(sk + n * D + 8 * c + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) dqv[4 * c + e] = fmaf(dl, kv[e], dqv[4 * c + e]);
            }
            if (second_order && wg != 0.f) {   // uniform: wg depends on (i, j) only
                const float dw = wave_sum(h == 0 ? dl : 0.f);   // this wave's 32 rows
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    dq2[e] = fmaf(dw, (float)sg2[(int64_t)j * D + lane + 64 * e], dq2[e]);
            }
        }
    }
    if (second_order) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) sdq2[wave][lane + 64 * e] = dq2[e];
        __syncthreads();
    }
    if (active) {
        const float c2 = second_order ? 1.f / (float)rows : 0.f;   // 2 * 1/2 * (1/n_i)
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 8 * c + 4 * h + e;
                float x = scale * dqv[4 * c + e];
                if (second_order) x = fmaf(scale * qv[4 * c + e] * c2, sdq2[0][d] + sdq2[1][d], x);
                dq[base + (int64_t)t * D + d] = store_cast<T>(x);
            }
    }
}

// ---------------------------------------------------------------- dH
// dH = sum_t c_t q'_t g_t^T over the rows of one chunk; thread (a, b) of the
// 16 x 16 grid owns the (D/16) x (D/16) tile at rows a*D/16, columns b*D/16.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dh_kernel(const T* __restrict__ q, const T* __restrict__ dout,
                                                          const f32x4_t* __restrict__ rowstat,
                                                          float* __restrict__ part, int Tn, int rows_per,
                                                          float scale) {
    constexpr int R = D / 16;
    __shared__ float sa[kSub * D];
    __shared__ float sb[kSub * D];
    const int tid = threadIdx.x;
    const int a = tid >> 4, b = tid & 15;
    const int64_t bh = blockIdx.y;
    const int P = gridDim.x;
    const int64_t base = bh * (int64_t)Tn * D;
    const int t0 = blockIdx.x * rows_per;
    const int t1 = min(Tn, t0 + rows_per);
    float acc[R][R];
#pragma unroll
    for (int x = 0; x < R; ++x)
#pragma unroll
        for (int y = 0; y < R; ++y) acc[x][y] = 0.f;
    for (int ts = t0; ts < t1; ts += kSub) {
        const int nh = min(kSub, t1 - ts);
        __syncthreads();
        for (int c = tid; c < nh * D; c += kThreads) {
            const int rr = c / D;
            const float cf = rowstat[bh * (int64_t)Tn + ts + rr][3];
            sa[c] = cf * scale * load_f32(q + base + (int64_t)ts * D + c);
            sb[c] = load_f32(dout + base + (int64_t)ts * D + c);
        }
        __syncthreads();
        for (int rr = 0; rr < nh; ++rr) {
            float xa[R], xb[R];
#pragma unroll
            for (int x = 0; x < R; ++x) {
                xa[x] = sa[rr * D + a * R + x];
                xb[x] = sb[rr * D + b * R + x];
            }
#pragma unroll
            for (int x = 0; x < R; ++x)
#pragma unroll
                for (int y = 0; y < R; ++y) acc[x][y] = fmaf(xa[x], xb[y], acc[x][y]);
        }
    }
    float* out = part + (bh * P + blockIdx.x) * (int64_t)D * D;
#pragma unroll
    for (int x = 0; x < R; ++x)
#pragma unroll
        for (int y = 0; y < R; ++y) out[(a * R + x) * D + b * R + y] = acc[x][y];
}

// dH (and, when dHT is given, its transpose) from the partial sums in fixed order.
__global__ __launch_bounds__(kThreads) void bwd_dh_reduce_kernel(const float* __restrict__ part,
                                                                 float* __restrict__ dH, float* __restrict__ dHT,
                                                                 int P, int D) {
    const int64_t bh = blockIdx.y;
    const int DD = D * D;
    const int e = blockIdx.x * kThreads + threadIdx.x;
    if (e >= DD) return;
    float s = 0.f;
    for (int p = 0; p < P; ++p) s += part[(bh * P + p) * (int64_t)DD + e];
    dH[bh * (int64_t)DD + e] = s;
    if (dHT) dHT[bh * (int64_t)DD + (e % D) * D + e / D] = s;
}

// ---------------------------------------------------------------- virt
// One wave per (bh, group of 16 KV blocks); threads 4u..4u+3 share block
// j = 16 x + u, thread p owning dims 16c + 4p + e. Visits every query row of
// every query block for which j is a virtual token.
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_virt_kernel(
    const T* __restrict__ q, const T* __restrict__ dout, const double* __restrict__ kbar,
    const float* __restrict__ vsum, const double* __restrict__ q2bar, const f32x4_t* __restrict__ rowstat,
    const uint32_t* __restrict__ mask, const float* __restrict__ wgate, float* __restrict__ dkb_out,
    float* __restrict__ dvh_out, float* __restrict__ dsg_out, int Tn, int N, int NW, float scale,
    int second_order) {
    constexpr int C = D / 16;
    constexpr int Q = D / 4;
    __shared__ __attribute__((aligned(16))) float sq[kVirtRows * D];
    __shared__ __attribute__((aligned(16))) float sg[kVirtRows * D];
    __shared__ f32x4_t srs[kVirtRows];
    __shared__ float sq2[D];

    const int tid = threadIdx.x;
    const int u = tid >> 2, p = tid & 3;
    const int64_t bh = blockIdx.y;
    const int j = blockIdx.x * kVirtBlocks + u;
    const bool valid = j < N;
    const int jc = valid ? j : N - 1;
    const int nj = min(kBlock, Tn - jc * kBlock);
    const int64_t base = bh * (int64_t)Tn * D;

    float kb[Q], vh[Q], dkb[Q], dvh[Q], dsg[Q];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t a = (bh * N + jc) * (int64_t)D + 16 * c + 4 * p + e;
            kb[4 * c + e] = (float)kbar[a];
            vh[4 * c + e] = vsum[a];
            dkb[4 * c + e] = dvh[4 * c + e] = dsg[4 * c + e] = 0.f;
        }

    for (int i = 0; i < N; ++i) {
        const bool use = valid && !bit_set(mask + (bh * N + i) * (int64_t)NW, jc);
        if (!__any(use)) continue;   // one wave: uniform
        const float wg = (second_order && use) ? wgate[(bh * N + i) * (int64_t)N + j] : 0.f;
        const int rows = min(kBlock, Tn - i * kBlock);
        float dw = 0.f;
        for (int s0 = 0; s0 < rows; s0 += kVirtRows) {
            const int nr = min(kVirtRows, rows - s0);
            const int64_t src = base + ((int64_t)i * kBlock + s0) * D;
            __syncthreads();
            for (int c = tid; c < nr * D; c += 64) {
                sq[c] = scale * load_f32(q + src + c);
                sg[c] = load_f32(dout + src + c);
            }
            if (tid < nr) srs[tid] = rowstat[bh * (int64_t)Tn + (int64_t)i * kBlock + s0 + tid];
            if (second_order && s0 == 0)
                for (int d = tid; d < D; d += 64) sq2[d] = (float)q2bar[(bh * N + i) * (int64_t)D + d];
            __syncthreads();
            for (int rr = 0; rr < nr; ++rr) {
                float zp = 0.f, gp = 0.f;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const f32x4_t a4 = lds4(sq + rr * D + 16 * c + 4 * p);
                    const f32x4_t b4 = lds4(sg + rr * D + 16 * c + 4 * p);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        zp = fmaf(a4[e], kb[4 * c + e], zp);
                        gp = fmaf(b4[e], vh[4 * c + e], gp);
                    }
                }
                zp += __shfl_xor(zp, 1);
                gp += __shfl_xor(gp, 1);
                zp += __shfl_xor(zp, 2);
                gp += __shfl_xor(gp, 2);
                const f32x4_t rs = srs[rr];
                const float a = use ? expf(zp + wg - rs[0]) : 0.f;
                const float dl = a * (gp + (float)nj * (rs[2] - rs[1]));
                dw += dl;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const f32x4_t a4 = lds4(sq + rr * D + 16 * c + 4 * p);
                    const f32x4_t b4 = lds4(sg + rr * D + 16 * c + 4 * p);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dkb[4 * c + e] = fmaf(dl, a4[e], dkb[4 * c + e]);
                        dvh[4 * c + e] = fmaf(a, b4[e], dvh[4 * c + e]);
                    }
                }
            }
        }
        if (second_order && use && wg != 0.f) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dsg[4 * c + e] = fmaf(0.5f * dw, sq2[16 * c + 4 * p + e], dsg[4 * c + e]);
        }
    }
    if (valid) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t a = (bh * N + j) * (int64_t)D + 16 * c + 4 * p + e;
                dkb_out[a] = dkb[4 * c + e];
                dvh_out[a] = dvh[4 * c + e];
                dsg_out[a] = dsg[4 * c + e];
            }
    }
}

// ---------------------------------------------------------------- kv
// One workgroup of 256 threads per (bh, KV block j); threads 4u..4u+3 share
// key row 64 j + u, thread p owning dims 16c + 4p + e.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_kv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ dout,
    const double* __restrict__ kbar, const float* __restrict__ vsum, const f32x4_t* __restrict__ rowstat,
    const uint32_t* __restrict__ mask, const float* __restrict__ dH, const float* __restrict__ dkb_v,
    const float* __restrict__ dvh_v, const float* __restrict__ dsg_v, T* __restrict__ dk, T* __restrict__ dv,
    int Tn, int N, int NW, float scale, int second_order, int first_order, int nsplit) {
    // dkb_v / dvh_v hold nsplit partial sums (consecutive [BH, N, D] arrays), added in order.
    constexpr int C = D / 16;
    constexpr int Q = D / 4;
    constexpr int LD = D + 4;                  // padded row stride of the chain's staging
    __shared__ __attribute__((aligned(16))) float pool[2 * kKvRows * LD];
    __shared__ __attribute__((aligned(16))) float sH[16 * LD];
    __shared__ __attribute__((aligned(16))) float svh[D];
    __shared__ float sblk[3 * D];
    __shared__ f32x4_t srs[kKvRows];
    float* sA = pool;                           // main loop: q' rows (stride D)
    float* sB = pool + kKvRows * D;             //            g rows  (stride D)

    const int tid = threadIdx.x;
    const int u = tid >> 2, p = tid & 3;
    const int64_t bh = blockIdx.y;
    const int j = blockIdx.x;
    const int row = j * kBlock + u;
    const bool kvalid = row < Tn;
    const int nj = min(kBlock, Tn - j * kBlock);
    const int64_t base = bh * (int64_t)Tn * D;

    float kk[Q], vv[Q], dkk[Q], dvv[Q];
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t a = base + (int64_t)row * D + 16 * c + 4 * p + e;
            kk[4 * c + e] = kvalid ? load_f32(k + a) : 0.f;
            vv[4 * c + e] = kvalid ? load_f32(v + a) : 0.f;
            dkk[4 * c + e] = dvv[4 * c + e] = 0.f;
        }

    // Exact pairs: every query block i whose exact set holds j.
    for (int i = 0; i < N; ++i) {
        if (!bit_set(mask + (bh * N + i) * (int64_t)NW, j)) continue;   // uniform
        const int rows = min(kBlock, Tn - i * kBlock);
        const int64_t src = base + (int64_t)i * kBlock * D;
        __syncthreads();
        for (int c = tid; c < rows * D; c += kThreads) {
            sA[c] = scale * load_f32(q + src + c);
            sB[c] = load_f32(dout + src + c);
        }
        if (tid < rows) srs[tid] = rowstat[bh * (int64_t)Tn + (int64_t)i * kBlock + tid];
        __syncthreads();
        for (int rr = 0; rr < rows; ++rr) {
            float zp = 0.f, dp = 0.f;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const f32x4_t a4 = lds4(sA + rr * D + 16 * c + 4 * p);
                const f32x4_t b4 = lds4(sB + rr * D + 16 * c + 4 * p);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zp = fmaf(a4[e], kk[4 * c + e], zp);
                    dp = fmaf(b4[e], vv[4 * c + e], dp);
                }
            }
            zp += __shfl_xor(zp, 1);
            dp += __shfl_xor(dp, 1);
            zp += __shfl_xor(zp, 2);
            dp += __shfl_xor(dp, 2);
            const f32x4_t rs = srs[rr];
            const float P = expf(zp - rs[0]);
            const float ds = P * (dp - rs[1]);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const f32x4_t a4 = lds4(sA + rr * D + 16 * c + 4 * p);
                const f32x4_t b4 = lds4(sB + rr * D + 16 * c + 4 * p);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dkk[4 * c + e] = fmaf(ds, a4[e], dkk[4 * c + e]);
                    dvv[4 * c + e] = fmaf(P, b4[e], dvv[4 * c + e]);
                }
            }
        }
    }

    // Chain terms of block j, added straight into dkk / dvv:
    //   dk += (dkbar_v - dH V-hat_j) / n_j + dH v + 2 dsig2_j (k - kbar_j) / n_j,
    //   dv += dV-hat_j + dH^T (k - kbar_j).
    const int64_t jb = (bh * N + j) * (int64_t)D;
    const float inv_n = 1.f / (float)nj;
    float* skc = pool;                  // (k - kbar_j) rows, stride LD
    float* svr = pool + kKvRows * LD;   // v rows, stride LD
    __syncthreads();
    // the block's dkbar, dV-hat (summed over the partials, in order) and dsig2, once
    for (int d = tid; d < D; d += kThreads) {
        const int64_t stride = (int64_t)gridDim.y * N * D;
        float sk_ = 0.f, sv_ = 0.f;
        for (int sp = 0; sp < nsplit; ++sp) {
            sk_ += dkb_v[sp * stride + jb + d];
            sv_ += dvh_v[sp * stride + jb + d];
        }
        sblk[d] = sk_;
        sblk[D + d] = sv_;
        sblk[2 * D + d] = second_order ? dsg_v[jb + d] : 0.f;
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * c + 4 * p + e;
            const int y = 4 * c + e;
            const float kc = kvalid ? kk[y] - (float)kbar[jb + d] : 0.f;
            skc[u * LD + d] = kc;
            svr[u * LD + d] = vv[y];
        }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int d = 16 * c + 4 * p + e;
            const int y = 4 * c + e;
            dkk[y] += sblk[d] * inv_n;
            if (second_order) dkk[y] = fmaf(2.f * sblk[2 * D + d] * inv_n, skc[u * LD + d], dkk[y]);
            dvv[y] += sblk[D + d];
        }
    for (int d = tid; d < D; d += kThreads) svh[d] = vsum[jb + d];
    if (first_order) {
        const float* dHm = dH + bh * (int64_t)D * D;
        for (int c = 0; c < C; ++c) {      // dH rows 16c .. 16c + 15
            __syncthreads();
            for (int x = tid; x < 16 * D; x += kThreads) sH[(x / D) * LD + x % D] = dHm[(int64_t)16 * c * D + x];
            __syncthreads();
            // dv_e += sum_d dH[d][e] (k - kbar)_d over the chunk's rows d (own e)
            for (int dd = 0; dd < 16; ++dd) {
                const float kc = skc[u * LD + 16 * c + dd];
#pragma unroll
                for (int c2 = 0; c2 < C; ++c2) {
                    const f32x4_t h4 = lds4(sH + dd * LD + 16 * c2 + 4 * p);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dvv[4 * c2 + e] = fmaf(h4[e], kc, dvv[4 * c2 + e]);
                }
            }
            // dk_d += sum_e dH[d][e] (v_e - V-hat_j,e / n_j) for the own rows d = 16c + 4p + e
            float xs[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* hr = sH + (4 * p + e) * LD;
                float s1 = 0.f, s2 = 0.f;
                for (int x = 0; x < D; x += 4) {
                    const f32x4_t h4 = lds4(hr + x);
                    const f32x4_t v4 = lds4(svr + u * LD + x);
                    const f32x4_t w4 = lds4(svh + x);
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        s1 = fmaf(h4[z], v4[z], s1);
                        s2 = fmaf(h4[z], w4[z], s2);
                    }
                }
                xs[e] = s1 - s2 * inv_n;
            }
            // c is a runtime index here: select the own registers by unrolled compare
#pragma unroll
            for (int cc = 0; cc < C; ++cc)
                if (cc == c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dkk[4 * cc + e] += xs[e];
        }
    }
    if (kvalid) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t a = base + (int64_t)row * D + 16 * c + 4 * p + e;
                dk[a] = store_cast<T>(dkk[4 * c + e]);
                dv[a] = store_cast<T>(dvv[4 * c + e]);
            }
    }
}

struct BwdLayout {
    size_t rowstat, mask, dkb, dvh, dsg, dhp, dh, dht, planes, dq2, dw, total;
    int NW, P, S;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// bf16 inputs add the matrix-core kernels' buffers: dH transposed, bf16 hi +
// lo planes of kbar, V-hat and H, dq2bar and the dW table.
BwdLayout bwd_layout(const Geom& g, bool mfma) {
    BwdLayout L;
    L.NW = (g.N + 31) / 32;
    L.P = dh_parts(g.T);
    L.S = mfma ? bwd_virt_splits(g) : 1;   // partial sums of dkbar, dV-hat over query ranges
    const size_t BH = (size_t)g.BH, ND = (size_t)g.N * g.D, DD = (size_t)g.D * g.D;
    size_t o = 0;
    L.rowstat = o; o = align256(o + BH * g.T * sizeof(f32x4_t));
    L.mask = o;    o = align256(o + BH * g.N * L.NW * sizeof(uint32_t));
    L.dkb = o;     o = align256(o + L.S * BH * ND * sizeof(float));
    L.dvh = o;     o = align256(o + L.S * BH * ND * sizeof(float));
    L.dsg = o;     o = align256(o + BH * ND * sizeof(float));
    L.dhp = o;     o = align256(o + BH * L.P * DD * sizeof(float));
    L.dh = o;      o = align256(o + BH * DD * sizeof(float));
    L.dht = o;     o = align256(o + (mfma ? BH * DD * sizeof(float) : 0));
    L.planes = o;  o = align256(o + (mfma ? BH * (4 * ND + 2 * DD) * sizeof(bf16_t) : 0));
    L.dq2 = o;     o = align256(o + (mfma ? BH * ND * sizeof(float) : 0));
    L.dw = o;      o = align256(o + (mfma ? BH * g.N * (size_t)g.N * sizeof(float) : 0));
    L.total = o;
    return L;
}

template <typename T, int D>
hipError_t run_bwd(const Geom& g, const pisa_params_t* p, const void* q, const void* k, const void* v,
                   const void* o, const void* dout, const StatsView* st, const int32_t* idx,
                   const float* wgate, const float* fwd_rstat, void* dq, void* dk, void* dv, void* ws,
                   hipStream_t stream) {
    constexpr bool kMfma = std::is_same<T, bf16_t>::value;
    const BwdLayout L = bwd_layout(g, kMfma);
    unsigned char* w = static_cast<unsigned char*>(ws);
    auto* rowstat = reinterpret_cast<f32x4_t*>(w + L.rowstat);
    auto* mask = reinterpret_cast<uint32_t*>(w + L.mask);
    auto* dkb = reinterpret_cast<float*>(w + L.dkb);
    auto* dvh = reinterpret_cast<float*>(w + L.dvh);
    auto* dsg = reinterpret_cast<float*>(w + L.dsg);
    auto* dhp = reinterpret_cast<float*>(w + L.dhp);
    auto* dh = reinterpret_cast<float*>(w + L.dh);
    const unsigned BH = (unsigned)g.BH;
    const T* tq = static_cast<const T*>(q);
    const T* tk = static_cast<const T*>(k);
    const T* tv = static_cast<const T*>(v);
    const T* to = static_cast<const T*>(o);
    const T* tg = static_cast<const T*>(dout);
    const int so = p->second_order, fo = p->first_order;

    hipLaunchKernelGGL(bwd_mask_kernel, dim3(g.N, BH), dim3(64), L.NW * sizeof(uint32_t), stream,
                       p->topk > 0 ? idx : nullptr, mask, g.N, L.NW, p->topk, p->band, p->n_sink);
    float* dht = kMfma ? reinterpret_cast<float*>(w + L.dht) : nullptr;
    if constexpr (kMfma) {
        bf16_t* pl = reinterpret_cast<bf16_t*>(w + L.planes);
        const size_t ND = (size_t)g.BH * g.N * D, DD = (size_t)g.BH * D * D;
        bf16_t *kbh = pl, *kbl = pl + ND, *vhh = pl + 2 * ND, *vhl = pl + 3 * ND;
        bf16_t *hh = pl + 4 * ND, *hl = pl + 4 * ND + DD;
        float* dw = reinterpret_cast<float*>(w + L.dw);
        const float* wg = so ? wgate : nullptr;
        hipError_t e = launch_bwd_prep(g, st, kbh, kbl, vhh, vhl, hh, hl, stream);
        if (e == hipSuccess)
            e = fwd_rstat ? launch_bwd_rowstats_fwd(g, tq, to, tg, hh, hl, fwd_rstat, rowstat, fo, stream)
                          : launch_bwd_rowstats(g, tq, tk, to, tg, kbh, kbl, hh, hl, mask, wg, rowstat, L.NW, so, fo,
                                                stream);
        if (e == hipSuccess)
            e = launch_bwd_virt_mfma(g, tq, tg, st, mask, rowstat, wg, dkb, dvh, dw, dsg, L.NW, so, stream);
        if (e == hipSuccess)
            e = launch_bwd_dq(g, tq, tk, tv, tg, kbh, kbl, vhh, vhl, hh, hl, mask, wg, rowstat, dw,
                              so ? st->ksig2 : nullptr, reinterpret_cast<float*>(w + L.dq2), static_cast<bf16_t*>(dq),
                              L.NW, so, fo, stream);
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((bwd_row_kernel<T, D>), dim3(g.N, BH), dim3(kRowThreads), L.NW * sizeof(uint32_t),
                           stream, tq, tk, tv, to, tg, st->kbar, st->vsum, so ? st->ksig2 : nullptr, st->hsum,
                           mask, so ? wgate : nullptr, static_cast<T*>(dq), rowstat, g.T, g.N, L.NW, g.scale, so,
                           fo);
        hipLaunchKernelGGL((bwd_virt_kernel<T, D>), dim3((g.N + kVirtBlocks - 1) / kVirtBlocks, BH), dim3(64), 0,
                           stream, tq, tg, st->kbar, st->vsum, so ? st->q2bar : nullptr, rowstat, mask,
                           so ? wgate : nullptr, dkb, dvh, dsg, g.T, g.N, L.NW, g.scale, so);
    }
    if (fo) {
        const int rows_per = (g.T + L.P - 1) / L.P;
        if constexpr (kMfma) {
            const hipError_t e = launch_bwd_dh_mfma(g, tq, tg, rowstat, dhp, L.P, stream);
            if (e != hipSuccess) return e;
        } else {
            hipLaunchKernelGGL((bwd_dh_kernel<T, D>), dim3(L.P, BH), dim3(kThreads), 0, stream, tq, tg, rowstat,
                               dhp, g.T, rows_per, g.scale);
        }
        hipLaunchKernelGGL(bwd_dh_reduce_kernel, dim3((D * D + kThreads - 1) / kThreads, BH), dim3(kThreads),
                           0, stream, dhp, dh, dht, L.P, D);
    }
    if constexpr (kMfma) {
        const hipError_t e = launch_bwd_dkdv(g, tq, tk, tv, tg, mask, rowstat, st, dh, dht, dkb, dvh, dsg,
                                             static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), L.NW, L.S, so, fo,
                                             stream);
        if (e != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((bwd_kv_kernel<T, D>), dim3(g.N, BH), dim3(kThreads), 0, stream, tq, tk, tv, tg,
                           st->kbar, st->vsum, rowstat, mask, dh, dkb, dvh, dsg, static_cast<T*>(dk),
                           static_cast<T*>(dv), g.T, g.N, L.NW, g.scale, so, fo, L.S);
    }
    return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(const Geom& g, int dtype) { return bwd_layout(g, dtype == PISA_BF16).total; }

hipError_t launch_attn_bwd(const Geom& g, int dtype, const pisa_params_t* p, const void* q, const void* k,
                           const void* v, const void* o, const void* dout, const StatsView* st,
                           const int32_t* idx, const float* wgate, const float* fwd_rstat, void* dq, void* dk,
                           void* dv, void* ws, hipStream_t stream) {
    if (dtype == PISA_BF16) {
        if (g.D == 128)
            return run_bwd<bf16_t, 128>(g, p, q, k, v, o, dout, st, idx, wgate, fwd_rstat, dq, dk, dv, ws, stream);
        return run_bwd<bf16_t, 64>(g, p, q, k, v, o, dout, st, idx, wgate, fwd_rstat, dq, dk, dv, ws, stream);
    }
    // fp32 inputs: the row kernel derives lse together with dq, so it recomputes them
    if (g.D == 128) return run_bwd<float, 128>(g, p, q, k, v, o, dout, st, idx, wgate, nullptr, dq, dk, dv, ws, stream);
    return run_bwd<float, 64>(g, p, q, k, v, o, dout, st, idx, wgate, nullptr, dq, dk, dv, ws, stream);
}

}  // namespace pisa
