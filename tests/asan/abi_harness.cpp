// Host-side exercise of libpisa's C ABI for the address and undefined-behaviour
// sanitizers: every entry point's validation paths (which return before any
// HIP call), the size and layout queries, the kernel plan and the host Z-order.
// Built with the library's host code only (no device code), run on any host;
// exits non-zero on a wrong status, the sanitizers abort on a defect.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pisa.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static void* fake(int n) { return (void*)(uintptr_t)((uint64_t)(n + 1) << 32); }   // distinct, never dereferenced

static pisa_shape_t shape(int64_t T, int64_t D, int dtype, int64_t H) {
    pisa_shape_t s;
    memset(&s, 0, sizeof s);
    s.batch = 1; s.heads = H; s.seq_len = T; s.head_dim = D; s.block_size = 64; s.dtype = dtype; s.scale = 0.f;
    return s;
}

static pisa_params_t params(int topk, int band, int so, int n_sink, int cov) {
    pisa_params_t p;
    memset(&p, 0, sizeof p);
    p.topk = topk; p.band = band; p.second_order = so; p.first_order = 1; p.phase_mask = 0;
    p.n_sink = n_sink; p.cov_bias = cov;
    return p;
}

int main(void) {
    EXPECT(pisa_abi_version() == PISA_ABI_VERSION);
    for (int c = 0; c <= 9; ++c) EXPECT(pisa_status_str((pisa_status_t)c) != NULL);

    // sizes and layouts over a range of shapes, valid and not
    const int64_t Ts[] = {0, 1, 63, 64, 65, 1000, 32760, 118800, 524288, 524289};
    const int64_t Ds[] = {32, 64, 128, 256};
    for (int ti = 0; ti < 10; ++ti)
        for (int di = 0; di < 4; ++di)
            for (int dt = -1; dt <= 2; ++dt) {
                pisa_shape_t s = shape(Ts[ti], Ds[di], dt, 24);
                const int64_t N = pisa_num_blocks(&s);
                const size_t ws = pisa_stats_workspace_bytes(&s), ob = pisa_operands_bytes(&s);
                const size_t bw = pisa_attn_bwd_workspace_bytes(&s);
                int64_t off[PISA_OPERAND_COUNT];
                const pisa_status_t st = pisa_operands_offsets(&s, off);
                if (N < 0) {
                    EXPECT(ws == 0 && ob == 0 && bw == 0 && st != PISA_OK);
                } else {
                    EXPECT(N == (Ts[ti] + 63) / 64 && ws > 0 && ob > 0 && bw > 0 && st == PISA_OK);
                    for (int i = 1; i < PISA_OPERAND_COUNT; ++i) EXPECT(off[i] >= off[i - 1] && off[i] % 256 == 0);
                    EXPECT((size_t)off[PISA_OPERAND_COUNT - 1] <= ob);
                }
            }
    EXPECT(pisa_num_blocks(NULL) == -1);

    // the kernel plan, including bands far beyond N and huge topk
    {
        pisa_shape_t s = shape(118800, 128, PISA_BF16, 24);
        const int bands[] = {0, 1, 5, 1856, 1857, 1 << 20, 0x7fffffff};
        for (int b = 0; b < 7; ++b)
            for (int so = 0; so <= 1; ++so) {
                pisa_params_t p = params(232, bands[b], so, 3, 0);
                int32_t kern = -1;
                int64_t items = -1;
                EXPECT(pisa_attn_fwd_plan(&s, &p, &kern, &items) == PISA_OK);
                EXPECT(kern >= 0 && kern <= 2 && items > 0);
            }
        pisa_params_t bad = params(1858, 1, 0, 0, 0);
        EXPECT(pisa_attn_fwd_plan(&s, &bad, NULL, NULL) == PISA_ERR_PARAM);
        EXPECT(pisa_attn_fwd_plan(NULL, &bad, NULL, NULL) == PISA_ERR_NULL);
    }

    // every entry point rejects bad arguments before touching the device
    pisa_shape_t s = shape(1000, 64, PISA_BF16, 2);
    pisa_params_t p = params(4, 1, 0, 0, 0);
    pisa_stats_t st;
    memset(&st, 0, sizeof st);
    st.qbar = (double*)fake(10); st.kbar = (double*)fake(11); st.vsum = (float*)fake(12); st.hsum = (float*)fake(13);
    void *q = fake(1), *k = fake(2), *v = fake(3), *o = fake(4), *ops = fake(20), *ws = fake(21);
    const size_t opsb = (size_t)1 << 31;
    void* mis = (char*)fake(5) + 4;
    EXPECT(pisa_block_stats(NULL, &p, q, k, v, &st, ops, opsb, ws, 1 << 30, NULL) == PISA_ERR_NULL);
    EXPECT(pisa_block_stats(&s, &p, mis, k, v, &st, ops, opsb, ws, 1 << 30, NULL) == PISA_ERR_ALIGN);
    EXPECT(pisa_block_stats(&s, &p, q, k, v, &st, ops, 16, ws, 1 << 30, NULL) == PISA_ERR_WORKSPACE);
    EXPECT(pisa_block_stats(&s, &p, q, k, v, &st, (char*)k + 256, opsb, ws, 1 << 30, NULL) == PISA_ERR_PARAM);
    EXPECT(pisa_block_stats_noalloc(&s, &p, q, NULL, v, &st, ops, opsb, NULL) == PISA_ERR_NULL);
    {
        pisa_shape_t big = shape(4096, 128, PISA_BF16, 1024);
        EXPECT(pisa_block_stats_noalloc(&big, &p, q, k, v, &st, ops, opsb, NULL) == PISA_ERR_WORKSPACE);
    }
    EXPECT(pisa_prepare_operands(&s, &p, NULL, &st, ops, opsb, NULL) == PISA_ERR_NULL);
    EXPECT(pisa_route_topk(&s, &p, &st, NULL, opsb, (int32_t*)fake(30), NULL, NULL) == PISA_ERR_NULL);
    {
        pisa_params_t cov = params(4, 1, 0, 0, 1);
        EXPECT(pisa_route_topk(&s, &cov, &st, ops, opsb, (int32_t*)fake(30), NULL, NULL) == PISA_ERR_NULL);
        pisa_params_t badcov = params(4, 1, 0, 0, 2);
        EXPECT(pisa_route_topk(&s, &badcov, &st, ops, opsb, (int32_t*)fake(30), NULL, NULL) == PISA_ERR_PARAM);
    }
    EXPECT(pisa_attn_fwd(&s, &p, q, k, v, &st, ops, opsb, (int32_t*)fake(30), NULL, q, NULL, NULL) == PISA_ERR_PARAM);
    EXPECT(pisa_attn_fwd(&s, &p, q, k, v, &st, ops, opsb, (int32_t*)fake(30), NULL, o, (float*)k, NULL) ==
           PISA_ERR_PARAM);
    EXPECT(pisa_attn_fwd_valu(&s, &p, q, k, v, NULL, ops, opsb, (int32_t*)fake(30), NULL, o, NULL, NULL) ==
           PISA_ERR_NULL);
    EXPECT(pisa_attn_bwd(&s, &p, q, k, v, o, fake(6), &st, (int32_t*)fake(30), NULL, NULL, fake(7), fake(7), fake(8),
                         ws, (size_t)1 << 40, NULL) == PISA_ERR_PARAM);
    EXPECT(pisa_reorder_gather(&s, (int32_t*)fake(31), q, (char*)q + 1024, NULL) == PISA_ERR_PARAM);
    EXPECT(pisa_reorder_scatter(&s, NULL, q, k, NULL) == PISA_ERR_NULL);

    // host Z-order: a permutation of every cell
    {
        const int64_t grids[][3] = {{21, 30, 52}, {33, 45, 80}, {3, 5, 7}, {1, 1, 1}};
        for (int gi = 0; gi < 4; ++gi) {
            const int64_t n = grids[gi][0] * grids[gi][1] * grids[gi][2] + 7;
            int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * n);
            char* seen = (char*)calloc(n, 1);
            EXPECT(pisa_z_order(grids[gi], 3, 7, perm, n) == PISA_OK);
            for (int64_t i = 0; i < n; ++i) {
                EXPECT(perm[i] >= 0 && perm[i] < n && !seen[perm[i]]);
                if (perm[i] >= 0 && perm[i] < n) seen[perm[i]] = 1;
            }
            for (int64_t i = 0; i < 7; ++i) EXPECT(perm[i] == i);
            EXPECT(pisa_z_order(grids[gi], 3, 7, perm, n - 1) == PISA_ERR_SHAPE);
            free(seen);
            free(perm);
        }
        const int64_t huge[2] = {(int64_t)1 << 31, 2};
        int32_t one;
        EXPECT(pisa_z_order(huge, 2, 0, &one, 1) == PISA_ERR_SHAPE);
    }
    if (failures) {
        fprintf(stderr, "%d expectation(s) failed\n", failures);
        return 1;
    }
    printf("abi harness: all expectations met\n");
    return 0;
}
